// api.cpp -- the C ABI of libka_attn: validation on the host, then one launch
// sequence on the caller's stream.  No allocation, no synchronisation; the only state
// is a thread-local copy of the last HIP error (plus, in the launchers, a per-device
// cache of the CU count kept in atomics and a per-thread cache of the last dense plan).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <utility>

#include "ka_attn.h"
#include "ka_kernels.hpp"

namespace {

thread_local int g_last_hip_error = 0;

ka_status hip_status(hipError_t e) {
  if (e == hipSuccess) return KA_OK;
  g_last_hip_error = (int)e;
  return KA_ERR_HIP;
}

constexpr size_t HD_ = 64;  // head dim of the differential path and its parameter rows

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// [p, p + n) and [q, q + m) overlap
bool overlap(const void* p, size_t n, const void* q, size_t m) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p), b = reinterpret_cast<uintptr_t>(q);
  return n && m && a < b + m && b < a + n;
}

// B*H*S*D*elem without overflowing 64 bits (and each tensor below 2^62 bytes).
bool tensor_bytes(int B, int H, int S, int D, size_t elem, size_t* out) {
  unsigned __int128 n = (unsigned __int128)(unsigned)B * (unsigned)H * (unsigned)S * (unsigned)D * elem;
  if (n >> 62) return false;
  *out = (size_t)n;
  return true;
}

// B*H*ceil(S/64) < 2^23: the query blocks of 64 rows over all (b, h), the unit every
// launch's one-dimensional grid is sized by (at most 512 work-items each)
bool grid_ok(int B, int H, int S) { return (long long)B * H * ((S + 63) / 64) < (1LL << 23); }

// wide: head dim 512 is accepted (bf16 only)
ka_status check_dense(ka_dtype dt, const void* q, const void* k, const void* v, void* o, int B, int H, int Sq,
                      int Sk, int D, float scale, size_t* qbytes, size_t* kbytes, bool wide = false) {
  if (!q || !k || !v || !o) return KA_ERR_NULL;
  if (B < 1 || H < 1 || Sq < 1 || Sk < 1 || D < 1) return KA_ERR_SHAPE;
  if (D != 64 && !(wide && D == 512 && dt == KA_BF16)) return KA_ERR_UNSUPPORTED;
  if (dt != KA_F32 && dt != KA_BF16) return KA_ERR_UNSUPPORTED;
  if (!std::isfinite(scale) || !(scale > 0.0f)) return KA_ERR_PARAM;
  const size_t e = dt == KA_F32 ? 4 : 2;
  if (!tensor_bytes(B, H, Sq, D, e, qbytes) || !tensor_bytes(B, H, Sk, D, e, kbytes)) return KA_ERR_SHAPE;
  // every launch has at most 512 work-items per 64 query rows of a (b, h) and one grid
  // dimension, so B*H*ceil(Sq/64) below 2^23 keeps its work-item count within 32 bits; key
  // tiles use 32-bit buffer offsets
  if (!grid_ok(B, H, Sq)) return KA_ERR_SHAPE;
  if ((long long)Sk * D * (long long)e + 2LL * 64 * D * (long long)e > 0x7fffffffLL) return KA_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return KA_ERR_ALIGN;
  if (overlap(o, *qbytes, q, *qbytes) || overlap(o, *qbytes, k, *kbytes) || overlap(o, *qbytes, v, *kbytes))
    return KA_ERR_ALIAS;
  return KA_OK;
}

// A [B][H][S][64] bf16 view with element strides (batch, head, token): checks that every
// stride is a non-negative multiple of 8 (16-byte rows), the token stride at least 64, one
// (b, h) slice within the kernels' 32-bit buffer offsets, and the whole extent within 2^62
// bytes.  *extent = bytes from the base to the end of the last row.
bool view_ok(const ka_layout& L, int B, int H, int S, size_t* extent) {
  if (L.batch < 0 || L.head < 0 || L.token < 64) return false;
  if ((L.batch | L.head | L.token) & 7) return false;
  const unsigned __int128 slice = ((unsigned __int128)(S - 1) * (unsigned long long)L.token + 64) * 2;
  if (slice > 0x7fffffffu) return false;
  const unsigned __int128 last = (unsigned __int128)(B - 1) * (unsigned long long)L.batch +
                                 (unsigned __int128)(H - 1) * (unsigned long long)L.head +
                                 (unsigned __int128)(S - 1) * (unsigned long long)L.token + 64;
  if ((last * 2) >> 62) return false;
  *extent = (size_t)(last * 2);
  return true;
}

// No two (b, h, s) rows of the view share an element: sorted by stride (dims of extent 1
// left out), each stride covers everything the smaller ones span.
bool view_injective(const ka_layout& L, int B, int H, int S) {
  struct D { long long stride, n; } d[3] = {{L.batch, B}, {L.head, H}, {L.token, S}};
  for (int i = 0; i < 3; ++i)
    for (int j = i + 1; j < 3; ++j)
      if (d[j].stride < d[i].stride) std::swap(d[i], d[j]);
  long long span = 64;  // one row
  for (const D& x : d) {
    if (x.n == 1) continue;
    if (x.stride < span) return false;
    span = x.stride * (x.n - 1) + span;
  }
  return true;
}

// Validates a differential call and fills *out.  dry: stop after the shape, parameter,
// layout and output checks and report the workspace bytes the call needs in *need (no
// workspace checks, *out untouched).
ka_status diff_build(ka_dtype dtype, const void* q1, const void* k1, const void* q2, const void* k2,
                            const void* v, void* o, int B, int H, int Sq, int Sk, int D, float scale, int window,
                            ka_qknorm qk_norm, const float* dyt_alpha, const float* dyt_gamma, const float* dyt_beta,
                            const float* rms_weight, float rms_eps, int rotary_dims, float rope_base,
                            const float* lambda, const uint8_t* v_keep, const ka_layout* layouts, void* workspace,
                            size_t workspace_bytes, bool dry, size_t* need_out, ka::DiffArgs* out) {
  if (qk_norm != KA_QKNORM_DYT && qk_norm != KA_QKNORM_RMS) return KA_ERR_UNSUPPORTED;
  if (!q1 || !k1 || !q2 || !k2 || !v || !o || !lambda) return KA_ERR_NULL;
  if (qk_norm == KA_QKNORM_DYT && (!dyt_alpha || !dyt_gamma || !dyt_beta)) return KA_ERR_NULL;
  if (qk_norm == KA_QKNORM_RMS && !rms_weight) return KA_ERR_NULL;
  if (B < 1 || H < 1 || Sq < 1 || Sk < 1 || D < 1 || Sq != Sk) return KA_ERR_SHAPE;
  if (D != 64 || dtype != KA_BF16) return KA_ERR_UNSUPPORTED;
  if (!std::isfinite(scale) || !(scale > 0.0f) || !std::isfinite(rope_base) || !(rope_base > 1.0f))
    return KA_ERR_PARAM;
  if (rotary_dims != 32 && rotary_dims != 64) return KA_ERR_PARAM;
  if (qk_norm == KA_QKNORM_RMS && (!std::isfinite(rms_eps) || !(rms_eps > 0.0f))) return KA_ERR_PARAM;
  const int S = Sq;
  size_t tb = 0;
  if (!tensor_bytes(B, H, S, D, 2, &tb)) return KA_ERR_SHAPE;
  if (!grid_ok(B, H, S)) return KA_ERR_SHAPE;
  // views of q1, k1, q2, k2, v, o: the given strides, or contiguous [B][H][S][64]
  ka_layout lay[6];
  size_t ext[6];
  for (int t = 0; t < 6; ++t) {
    lay[t] = layouts ? layouts[t] : ka_layout{(int64_t)H * S * 64, (int64_t)S * 64, 64};
    if (!view_ok(lay[t], B, H, S, &ext[t])) return KA_ERR_SHAPE;
  }
  if (!view_injective(lay[5], B, H, S)) return KA_ERR_SHAPE;  // rows of o written twice
  const void* ins[5] = {q1, k1, q2, k2, v};
  for (const void* p : ins)
    if (!aligned16(p)) return KA_ERR_ALIGN;
  if (!aligned16(o)) return KA_ERR_ALIGN;
  const size_t need = ka::diff_workspace_bytes(B, H, S, window, v_keep != nullptr);
  *need_out = need;
  // o against the extents [base, base + ext) of the input views (inputs may share memory with
  // each other), the V flags and the parameter arrays, which every workgroup reads while others
  // write o
  const void* prm[5] = {dyt_alpha, dyt_gamma, dyt_beta, rms_weight, lambda};
  const size_t prm_bytes[5] = {4 * sizeof(float), 4 * HD_ * sizeof(float), 4 * HD_ * sizeof(float),
                               4 * HD_ * sizeof(float), (size_t)H * sizeof(float)};
  const bool prm_used[5] = {qk_norm == KA_QKNORM_DYT, qk_norm == KA_QKNORM_DYT, qk_norm == KA_QKNORM_DYT,
                            qk_norm == KA_QKNORM_RMS, true};
  const size_t nk = v_keep ? (size_t)B * S : 0;
  for (int t = 0; t < 5; ++t)
    if (overlap(o, ext[5], ins[t], ext[t])) return KA_ERR_ALIAS;
  if (overlap(o, ext[5], v_keep, nk)) return KA_ERR_ALIAS;
  for (int t = 0; t < 5; ++t)
    if (prm_used[t] && overlap(o, ext[5], prm[t], prm_bytes[t])) return KA_ERR_ALIAS;
  if (dry) return KA_OK;
  if (need) {
    if (!workspace) return KA_ERR_NULL;
    if (workspace_bytes < need) return KA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return KA_ERR_ALIGN;
    // the workspace against o, the inputs, the V flags and the parameter arrays
    if (overlap(o, ext[5], workspace, need)) return KA_ERR_ALIAS;
    for (int t = 0; t < 5; ++t)
      if (overlap(workspace, need, ins[t], ext[t])) return KA_ERR_ALIAS;
    if (overlap(workspace, need, v_keep, nk)) return KA_ERR_ALIAS;
    for (int t = 0; t < 5; ++t)
      if (prm_used[t] && overlap(workspace, need, prm[t], prm_bytes[t])) return KA_ERR_ALIAS;
  }

  ka::DiffArgs& a = *out;
  std::memset(&a, 0, sizeof(a));
  a.q1 = static_cast<const unsigned short*>(q1);
  a.k1 = static_cast<const unsigned short*>(k1);
  a.q2 = static_cast<const unsigned short*>(q2);
  a.k2 = static_cast<const unsigned short*>(k2);
  a.v = static_cast<const unsigned short*>(v);
  a.o = static_cast<unsigned short*>(o);
  a.ws = static_cast<_Float16*>(workspace);
  a.alpha = dyt_alpha;
  a.gamma = dyt_gamma;
  a.beta = dyt_beta;
  a.rms_w = rms_weight;
  a.lambda = lambda;
  a.v_keep = v_keep;
  a.norm = qk_norm == KA_QKNORM_RMS ? 1 : 0;
  a.rms_eps = rms_eps;
  a.rot32 = rotary_dims == 32;
  a.B = B;
  a.H = H;
  a.S = S;
  for (int t = 0; t < 6; ++t) {
    a.sb[t] = lay[t].batch;
    a.sh[t] = lay[t].head;
    a.st[t] = (int)lay[t].token;
  }
  a.window = window < 0 ? -1 : window;
  a.c = scale * 1.4426950408889634f;
  const double two_pi = 6.283185307179586476925286766559;
  // positions need ceil(log2 S) bits; rev_hi keeps 24 - that many significant bits so
  // that p * rev_hi is exact in fp32, and rev_lo carries the rest
  int pbits = 1;
  while ((1 << pbits) < S) ++pbits;
  a.split_angles = pbits <= 16;
  // pair i: 64 rotary dims pair (i, i+32) for i < 32; 32 rotary dims pair (i, i+16) for
  // i < 16 at base^(-2i/32), and the threads' pairs 16..31 hold unrotated dims (angle 0)
  for (int i = 0; i < 32; ++i) {
    const double r = rotary_dims == 64 ? std::pow((double)rope_base, -2.0 * i / 64.0) / two_pi
                     : i < 16         ? std::pow((double)rope_base, -2.0 * i / 32.0) / two_pi
                                      : 0.0;
    a.rev[i] = r;
    int ex = 0;
    std::frexp(r, &ex);                                // r = m * 2^ex, 0.5 <= m < 1 (r = 0: 0)
    const double q = std::ldexp(1.0, ex - (24 - pbits));
    const double hi = std::round(r / q) * q;           // 24 - pbits significant bits
    a.rev_hi[i] = (float)hi;
    a.rev_lo[i] = (float)(r - hi);
  }
  return KA_OK;
}

}  // namespace

extern "C" {

ka_status ka_attn_fwd(ka_dtype dtype, const void* q, const void* k, const void* v, void* o, int B, int H, int Sq,
                      int Sk, int D, float scale, hipStream_t stream) {
  size_t qb = 0, kb = 0;
  ka_status st = check_dense(dtype, q, k, v, o, B, H, Sq, Sk, D, scale, &qb, &kb, true);
  if (st != KA_OK) return st;
  if (D == 512)
    return hip_status(ka::launch_attn512_bf16(static_cast<const unsigned short*>(q),
                                              static_cast<const unsigned short*>(k),
                                              static_cast<const unsigned short*>(v), static_cast<unsigned short*>(o),
                                              B, H, Sq, Sk, scale, stream));
  if (dtype == KA_F32)
    return hip_status(ka::launch_attn_f32(static_cast<const float*>(q), static_cast<const float*>(k),
                                          static_cast<const float*>(v), static_cast<float*>(o), B, H, Sq, Sk, scale,
                                          stream));
  return hip_status(ka::launch_attn_bf16(static_cast<const unsigned short*>(q), static_cast<const unsigned short*>(k),
                                         static_cast<const unsigned short*>(v), static_cast<unsigned short*>(o), B, H,
                                         Sq, Sk, scale, stream));
}

ka_status ka_xattn_fwd(ka_dtype dtype, const void* q, const void* k, const void* v, void* o, int B, int H, int Sq,
                       int Sk, int D, float scale, hipStream_t stream) {
  size_t qb = 0, kb = 0;
  ka_status st = check_dense(dtype, q, k, v, o, B, H, Sq, Sk, D, scale, &qb, &kb);
  if (st != KA_OK) return st;
  if (dtype == KA_BF16 && Sk > KA_XATTN_MAX_SK)  // too many keys to hold on chip: stream them in tiles
    return hip_status(ka::launch_attn_bf16(static_cast<const unsigned short*>(q), static_cast<const unsigned short*>(k),
                                           static_cast<const unsigned short*>(v), static_cast<unsigned short*>(o), B,
                                           H, Sq, Sk, scale, stream));
  if (dtype == KA_F32)
    return hip_status(ka::launch_attn_f32(static_cast<const float*>(q), static_cast<const float*>(k),
                                          static_cast<const float*>(v), static_cast<float*>(o), B, H, Sq, Sk, scale,
                                          stream));
  return hip_status(ka::launch_xattn_bf16(static_cast<const unsigned short*>(q), static_cast<const unsigned short*>(k),
                                          static_cast<const unsigned short*>(v), static_cast<unsigned short*>(o), B,
                                          H, Sq, Sk, scale, stream));
}

size_t ka_diffattn_workspace_bytes(int B, int H, int S, int D, int window) {
  size_t n = 0;
  if (B < 1 || H < 1 || S < 1 || D != 64 || !tensor_bytes(B, H, S, D, 2, &n)) return 0;
  return ka::diff_workspace_bytes(B, H, S, window, true);  // enough with or without V flags
}

ka_status ka_diffattn_fwd_ex(ka_dtype dtype, const void* q1, const void* k1, const void* q2, const void* k2,
                             const void* v, void* o, int B, int H, int Sq, int Sk, int D, float scale, int window,
                             ka_qknorm qk_norm, const float* dyt_alpha, const float* dyt_gamma,
                             const float* dyt_beta, const float* rms_weight, float rms_eps, int rotary_dims,
                             float rope_base, const float* lambda, const uint8_t* v_keep, const ka_layout* layouts,
                             void* workspace, size_t workspace_bytes, hipStream_t stream) {
  ka::DiffArgs a;
  size_t need = 0;
  const ka_status st = diff_build(dtype, q1, k1, q2, k2, v, o, B, H, Sq, Sk, D, scale, window, qk_norm, dyt_alpha,
                                  dyt_gamma, dyt_beta, rms_weight, rms_eps, rotary_dims, rope_base, lambda, v_keep,
                                  layouts, workspace, workspace_bytes, false, &need, &a);
  if (st != KA_OK) return st;
  return hip_status(ka::launch_diffattn(a, stream));
}

ka_status ka_diffattn_fwd_noalloc(ka_dtype dtype, const void* q1, const void* k1, const void* q2, const void* k2,
                                  const void* v, void* o, int B, int H, int Sq, int Sk, int D, float scale,
                                  int window, ka_qknorm qk_norm, const float* dyt_alpha, const float* dyt_gamma,
                                  const float* dyt_beta, const float* rms_weight, float rms_eps, int rotary_dims,
                                  float rope_base, const float* lambda, const uint8_t* v_keep,
                                  const ka_layout* layouts, hipStream_t stream) {
  size_t need = 0;
  ka_status st = diff_build(dtype, q1, k1, q2, k2, v, o, B, H, Sq, Sk, D, scale, window, qk_norm, dyt_alpha,
                            dyt_gamma, dyt_beta, rms_weight, rms_eps, rotary_dims, rope_base, lambda, v_keep, layouts,
                            nullptr, 0, true, &need, nullptr);
  if (st != KA_OK) return st;
  if (need > KA_STATIC_WORKSPACE_BYTES) return KA_ERR_WORKSPACE;  // before any HIP call
  void* ws = nullptr;
  size_t ws_bytes = 0;
  if (need) {
    const hipError_t e = ka::diff_static_workspace(&ws, &ws_bytes);
    if (e != hipSuccess) return hip_status(e);
  }
  ka::DiffArgs a;
  st = diff_build(dtype, q1, k1, q2, k2, v, o, B, H, Sq, Sk, D, scale, window, qk_norm, dyt_alpha, dyt_gamma,
                  dyt_beta, rms_weight, rms_eps, rotary_dims, rope_base, lambda, v_keep, layouts, ws, ws_bytes, false,
                  &need, &a);
  if (st != KA_OK) return st;
  return hip_status(ka::launch_diffattn(a, stream));
}

ka_status ka_diffattn_fwd(ka_dtype dtype, const void* q1, const void* k1, const void* q2, const void* k2,
                          const void* v, void* o, int B, int H, int Sq, int Sk, int D, float scale, int window,
                          const float* dyt_alpha, const float* dyt_gamma, const float* dyt_beta, float rope_base,
                          const float* lambda, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!dyt_alpha || !dyt_gamma || !dyt_beta) return KA_ERR_NULL;
  return ka_diffattn_fwd_ex(dtype, q1, k1, q2, k2, v, o, B, H, Sq, Sk, D, scale, window, KA_QKNORM_DYT, dyt_alpha,
                            dyt_gamma, dyt_beta, nullptr, 1.0f, 64, rope_base, lambda, nullptr, nullptr, workspace,
                            workspace_bytes, stream);
}

const char* ka_attn_kernel_name(ka_dtype dtype, int B, int H, int Sq, int Sk, int D) {
  if (B < 1 || H < 1 || Sq < 1 || Sk < 1 || !grid_ok(B, H, Sq)) return nullptr;
  if (dtype == KA_F32 && D == 64) return "attn_f32";
  if (dtype != KA_BF16) return nullptr;
  if (D == 512) return "attn512_pair";
  if (D != 64) return nullptr;
  return ka::attn_bf16_kernel_name(B, H, Sq);
}

const char* ka_status_string(ka_status s) {
  switch (s) {
    case KA_OK: return "ok";
    case KA_ERR_NULL: return "null pointer";
    case KA_ERR_SHAPE: return "invalid shape";
    case KA_ERR_UNSUPPORTED: return "unsupported head dim or dtype";
    case KA_ERR_PARAM: return "invalid scalar parameter";
    case KA_ERR_ALIGN: return "pointer not 16-byte aligned";
    case KA_ERR_ALIAS: return "output overlaps an input or the workspace";
    case KA_ERR_WORKSPACE: return "workspace too small";
    case KA_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

int ka_last_hip_error(void) { return g_last_hip_error; }

const char* ka_version(void) { return "0.1.0"; }

}  // extern "C"
