// ka_kernels.hpp -- launchers of the gfx950 kernels (internal to the library).
// Each launcher enqueues on `s` and returns hipGetLastError(); shapes were
// validated by the C ABI layer.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>

namespace ka {

hipError_t launch_attn_f32(const float* q, const float* k, const float* v, float* o, int B, int H, int Sq, int Sk,
                           float scale, hipStream_t s);
hipError_t launch_attn_bf16(const unsigned short* q, const unsigned short* k, const unsigned short* v,
                            unsigned short* o, int B, int H, int Sq, int Sk, float scale, hipStream_t s);
// name and layout of the kernel launch_attn_bf16 picks for this shape on the current device
const char* attn_bf16_kernel_name(int B, int H, int Sq);
// head dim 512 (one kernel, bf16): the SDXL VAE's single-head attention
hipError_t launch_attn512_bf16(const unsigned short* q, const unsigned short* k, const unsigned short* v,
                               unsigned short* o, int B, int H, int Sq, int Sk, float scale, hipStream_t s);
hipError_t launch_xattn_bf16(const unsigned short* q, const unsigned short* k, const unsigned short* v,
                             unsigned short* o, int B, int H, int Sq, int Sk, float scale, hipStream_t s);

// Everything the differential kernels need, passed by value.
struct DiffArgs {
  const unsigned short* q1;
  const unsigned short* k1;
  const unsigned short* q2;
  const unsigned short* k2;
  const unsigned short* v;
  unsigned short* o;
  _Float16* ws;            // full path: k1^, k2^ [2][B][H][S][64] fp16, then (with v_keep) flagged V bf16
  const float* alpha;      // [4]      DyT
  const float* gamma;      // [4][64]  DyT
  const float* beta;       // [4][64]  DyT
  const float* rms_w;      // [4][64]  RMSNorm weight
  const float* lambda;     // [H]
  const unsigned char* v_keep;  // [B][S] or null: a 0 flag zeroes that token's V row
  int norm;                // 0: DyT, 1: RMSNorm
  float rms_eps;
  int rot32;               // 1: rotary on dims 0..31 (pairs i, i+16), dims 32..63 unrotated
  int B, H, S;
  // element strides of q1, k1, q2, k2, v, o (in that order) as [B][H][S][64] views: batch,
  // head and token; the 64 dims of a token are contiguous
  long long sb[6], sh[6];
  int st[6];
  int window;              // >= 0: |i - j| <= window; < 0: all keys
  float c;                 // scale * log2(e)
  double rev[32];          // revolutions per position of pair i: rope_base^(-2i/64) / (2 pi), or with
                           // rot32 rope_base^(-2i/32) / (2 pi) for i < 16 and 0 (no rotation) above
  float rev_hi[32];        // rev split for fp32 angle reduction: rev_hi * p exact for p < 2^split_bits
  float rev_lo[32];
  int split_angles;        // 1: S <= 2^16, use rev_hi/rev_lo; 0: fp64 angles
};

// Largest window the one-pass band kernel takes; wider windows use the flash path.
constexpr int BAND_MAX_WINDOW = 40;

size_t diff_workspace_bytes(int B, int H, int S, int window, bool v_flags);
// The allocation-free workspace of ka_diffattn_fwd_noalloc: this device's copy of a file-scope
// device array of KA_STATIC_WORKSPACE_BYTES; its address is looked up once per device.
hipError_t diff_static_workspace(void** ptr, size_t* bytes);
hipError_t launch_diffattn(const DiffArgs& a, hipStream_t s);

}  // namespace ka
