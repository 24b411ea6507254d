// ka_common.hpp -- building blocks shared by the gfx950 attention kernels.
//
// Matrix-core conventions (v_mfma_f32_16x16x32_{bf16,f16}, wave64), as used by
// every kernel here:
//   A (16 x 32): lane l holds row l%16, k = 8*(l/16) + e   (e = 0..7)
//   B (32 x 16): lane l holds column l%16, k = 8*(l/16) + e
//   C (16 x 16): lane l holds column l%16, rows 4*(l/16) + e (e = 0..3)
// The kernels compute S^T = K Q^T and O^T = V^T P^T so that one lane owns one
// query column: the softmax statistics of a query live in a single lane group
// and the rescale of O is a per-lane scalar.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ka {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(4))) _Float16 f16x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int HD = 64;                 // head dim this library is built for
constexpr float LOG2E = 1.4426950408889634f;

__device__ __forceinline__ f32x4 mfma_bf16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f16(const f16x8& a, const f16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Reduction over the four lanes {l, l^16, l^32, l^48} (the four row groups of a
// C tile that hold the same query column).  permlane16_swap(x, x) yields the
// even-row and odd-row copies of each 16-lane pair; permlane32_swap(x, x) the
// lower and upper halves.
__device__ __forceinline__ float group4_max(float x) {
  u32x2 a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  float y = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  u32x2 b = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float group4_sum(float x) {
  u32x2 a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  u32x2 b = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Sum over the four consecutive lanes {4k .. 4k+3} (DPP quad permutations [1,0,3,2],
// then [2,3,0,1]); every lane of the quad gets the same value.
__device__ __forceinline__ float quad_sum(float x) {
  const float y = x + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, true));
  return y + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(y), 0x4E, 0xF, 0xF, true));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Lazily raised running maximum of the online softmax: the reference maximum moves
// only when a tile's maximum exceeds it by more than LAZY_LOG2 in the exp2 domain;
// until then the weights are taken against the stale maximum (they stay below
// 2^LAZY_LOG2, far inside fp32 and bf16 range) and O is not rescaled.  O / l is
// unchanged in exact arithmetic: both carry the same factor.
constexpr float LAZY_LOG2 = 8.0f;

// Pin a value in an fp32 register: the empty asm is opaque to the optimizer, so the
// producing multiply cannot be contracted into a consumer (an FMA, or a mixed-
// precision v_fma_mix that rounds once to fp16).  Used where two code paths must
// round identically.
__device__ __forceinline__ float pin(float x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Transposed LDS read (ds_read_b64_tr_b16).  Within each 16-lane group, lane i
// receives slot e = element (i%4) of the 8 bytes addressed by source lane 4e + i/4.
// With source lane s pointing at row r(s/4), column c0 + 4*(s%4) of a row-major
// 16-bit matrix, lane i gets column c0 + i of rows r(0..3).
__device__ __forceinline__ i16x4 lds_read_tr16(const void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
}

__device__ __forceinline__ bf16x8 cat_bf16(i16x4 lo, i16x4 hi) {
  bf16x8 r;
  bf16x4 a = __builtin_bit_cast(bf16x4, lo), b = __builtin_bit_cast(bf16x4, hi);
  r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
  r[4] = b[0]; r[5] = b[1]; r[6] = b[2]; r[7] = b[3];
  return r;
}

// Pack 4 + 4 fp32 values into one bf16x8 MFMA operand (round to nearest even).
__device__ __forceinline__ bf16x8 pack_bf16(const f32x4& lo, const f32x4& hi) {
  bf16x8 r;
  r[0] = (__bf16)lo[0]; r[1] = (__bf16)lo[1]; r[2] = (__bf16)lo[2]; r[3] = (__bf16)lo[3];
  r[4] = (__bf16)hi[0]; r[5] = (__bf16)hi[1]; r[6] = (__bf16)hi[2]; r[7] = (__bf16)hi[3];
  return r;
}

__device__ __forceinline__ float bf16_bits_to_f32(unsigned short b) { return __uint_as_float((unsigned)b << 16); }

// Buffer resource over [base, base + bytes): raw buffer loads past `bytes` return
// zero without touching memory, so tile loads need no per-lane branch.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int RSRC_FLAGS = 0x00020000;  // dword 3 of a raw (untyped) buffer descriptor
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, RSRC_FLAGS);
}
__device__ __forceinline__ unsigned buf_ld1(rsrc_t r, int byte_offset) {
  return __builtin_amdgcn_raw_buffer_load_b8(r, byte_offset, 0, 0);
}
__device__ __forceinline__ uint4 buf_ld16(rsrc_t r, int byte_offset) {
  typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, byte_offset, 0, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// ---- direct global-to-LDS tile loads into unpadded, XOR-swizzled rings of 128-byte rows: chunk
// c (16 bytes) of ring row r sits at chunk position c ^ swz(r), so that fragment reads hit
// distinct banks.
// K: a b128 fragment read takes one chunk of 16 consecutive rows; rows 2m, 2m + 1 share a
// position and fall in the two 128-byte halves of the banks, the 8 pairs in 8 positions.
__device__ __forceinline__ int swz_k(int r) { return (r >> 1) & 7; }
// V: the transposed reads take 8-byte halves of one chunk from rows 4 apart.
__device__ __forceinline__ int swz_v(int r) { return ((r >> 1) & 3) << 1; }

typedef __attribute__((ext_vector_type(4))) unsigned u32x4_t;
// The four words of a raw buffer descriptor (the format make_rsrc builds), in scalar registers.
__device__ __forceinline__ u32x4_t raw_rsrc(const void* base, int bytes) {
  const unsigned long long p = (unsigned long long)base;
  u32x4_t r;
  r[0] = __builtin_amdgcn_readfirstlane((unsigned)p);
  r[1] = __builtin_amdgcn_readfirstlane((unsigned)(p >> 32) & 0xffffu);
  r[2] = __builtin_amdgcn_readfirstlane((unsigned)bytes);
  r[3] = RSRC_FLAGS;
  return r;
}
// The same buffer moved on by off bytes (off >= 0, wave-uniform): the base advanced and the size
// shrunk, to zero past the end, so offsets past the end still read zeros.  Scalar arithmetic, so
// that a loop can step a tile offset without a per-lane add.
__device__ __forceinline__ u32x4_t rsrc_advance(u32x4_t r, unsigned off) {
  const unsigned long long b = ((unsigned long long)r[1] << 32 | r[0]) + off;
  // every word through readfirstlane: the descriptor operand must stay in scalar registers
  u32x4_t n;
  n[0] = __builtin_amdgcn_readfirstlane((unsigned)b);
  n[1] = __builtin_amdgcn_readfirstlane((unsigned)(b >> 32));
  const int rem = (int)r[2] - (int)off;  // buffers stay below 2 GiB
  n[2] = __builtin_amdgcn_readfirstlane(rem > 0 ? rem : 0);
  n[3] = r[3];
  return n;
}
// 16 bytes per lane from the buffer (offsets past its size read as zero) straight into LDS, lane l's
// bytes at lds_base + 16 l.  M0 carries the wave's LDS base and is restored afterwards.  Inline
// assembly, so that the compiler does not make every later LDS read wait for the load: the caller
// waits (s_waitcnt) right before the barrier that publishes the data.
__device__ __forceinline__ void load16_to_lds(u32x4_t rsrc, int voff, unsigned lds_base) {
  unsigned saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds\n\ts_mov_b32 m0, %0"
               : "=&s"(saved)
               : "v"(voff), "s"(rsrc), "s"(lds_base)
               : "memory");
}
__device__ __forceinline__ unsigned lds_addr(const unsigned short* p) {
  return __builtin_amdgcn_readfirstlane((unsigned)(size_t)(__attribute__((address_space(3))) const unsigned short*)p);
}

// Scheduling-group masks for __builtin_amdgcn_sched_group_barrier.
constexpr int SG_VALU = 0x002, SG_MFMA = 0x008, SG_VMEM_READ = 0x020, SG_DS_READ = 0x100, SG_DS_WRITE = 0x200,
              SG_TRANS = 0x400;

// 16-byte global load / store helpers.
__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ void st16(void* p, const uint4& v) { *reinterpret_cast<uint4*>(p) = v; }
__device__ __forceinline__ void st8(void* p, const uint2& v) { *reinterpret_cast<uint2*>(p) = v; }
__device__ __forceinline__ uint2 ld8(const void* p) { return *reinterpret_cast<const uint2*>(p); }

// Unpack 8 bf16 (one uint4) into fp32.
__device__ __forceinline__ void unpack_bf16x8(const uint4& u, float* f) {
  const unsigned w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

// Unpack 4 bf16 (one uint2) into fp32.
__device__ __forceinline__ void unpack_bf16x4(const uint2& u, float* f) {
  f[0] = __uint_as_float(u.x << 16);
  f[1] = __uint_as_float(u.x & 0xffff0000u);
  f[2] = __uint_as_float(u.y << 16);
  f[3] = __uint_as_float(u.y & 0xffff0000u);
}

// Four fp32 -> four bf16 packed into 8 bytes.
__device__ __forceinline__ uint2 pack4_bf16_bits(float a, float b, float c, float d) {
  bf16x4 v;
  v[0] = (__bf16)a; v[1] = (__bf16)b; v[2] = (__bf16)c; v[3] = (__bf16)d;
  return __builtin_bit_cast(uint2, v);
}

// Store one 16-query x 64-dim output tile held in the O^T C layout (lane: query l % 16, dims
// 16 db + 4 (l / 16) + e) as 16 contiguous bytes per lane: one v_permlane16_swap per register
// trades dims between the lane groups l / 16 = 0, 1 (and 2, 3), so that group g holds dims
// 8 (g >> 1) + 16 (g & 1) + 32 h .. + 7 for h = 0, 1; a store instruction then writes 64
// contiguous bytes of each row.  row_ptr: the lane's output row (dims 0..63); ok: row exists.
// Every lane of the wave calls it (the swap reads the partner lane's registers); the four lanes
// of a query share its ok, so values only move between lanes that store together or not at all.
__device__ __forceinline__ void store_tile_rows(unsigned short* row_ptr, bool ok, int grp, const uint2 (&p)[4]) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint2 x = p[2 * h], y = p[2 * h + 1];
    const u32x2 s0 = __builtin_amdgcn_permlane16_swap(x.x, y.x, false, false);
    const u32x2 s1 = __builtin_amdgcn_permlane16_swap(x.y, y.y, false, false);
    // s?[0]: the new first operand (own dims in groups 0 and 2, the partner's in 1 and 3),
    // s?[1]: the new second operand (the partner's in groups 0 and 2, own in 1 and 3)
    const uint4 v = make_uint4(s0[0], s1[0], s0[1], s1[1]);
    if (ok) st16(row_ptr + 32 * h + 8 * (grp >> 1) + 16 * (grp & 1), v);
  }
}

// DyT: gamma * tanh(alpha x) + beta.  With tanh(y) = 1 - 2/(1 + e^{2y}) this is
// (gamma + beta) - 2 gamma / (1 + e^{2 alpha x}): one exp, one reciprocal, one FMA,
// given k2a = 2 log2(e) alpha, gpb = gamma + beta and m2g = -2 gamma.  It saturates
// correctly: e^{2y} -> inf gives gamma + beta, e^{2y} -> 0 gives beta - gamma.
__device__ __forceinline__ float dyt(float x, float k2a, float gpb, float m2g) {
  const float e = fast_exp2(k2a * x);
  return __builtin_fmaf(m2g, __builtin_amdgcn_rcpf(1.0f + e), gpb);
}

// Rotary angle of position p for one frequency, as cos/sin.  The angle in
// revolutions, p * F (F = f / (2 pi)), is reduced to a small range before the
// hardware sin/cos (which take revolutions): an fp32 product p * F at p ~ 2e4
// would be off by ~1e-3 rad.
//  split form (positions below 2^16): F = fhi + flo with fhi short enough that
//    p * fhi is exact in fp32; u = (p fhi - rint(p fhi)) + p flo.
//  fp64 form (longer sequences): u = p F - rint(p F) in double.
__device__ __forceinline__ void rope_cs_split(float pf, float fhi, float flo, float& c, float& s) {
  const float t = pf * fhi;
  const float u = __builtin_fmaf(pf, flo, t - __builtin_rintf(t));
  c = __builtin_amdgcn_cosf(u);
  s = __builtin_amdgcn_sinf(u);
}
__device__ __forceinline__ void rope_cs_f64(int p, double rev_per_pos, float& c, float& s) {
  double t = (double)p * rev_per_pos;
  t -= __builtin_rint(t);
  const float f = (float)t;
  c = __builtin_amdgcn_cosf(f);
  s = __builtin_amdgcn_sinf(f);
}

}  // namespace ka
