// diffattn.hip -- fused differential attention with DyT and rotary embedding, gfx950.
//
// Method ("401 -> 163 ms: Stable Audio 3 medium on one TPU v6e chip", s3, s5,
// appendix E1, E2, D4): read the q/k/v projections once; normalise q and k with
// DyT in fp32 (s2: bf16 DyT flips the winning key of a near-argmax softmax);
// rotate them (rotate-half rotary embedding); run two softmax branches that
// weight the same V; subtract lambda times branch 2 from branch 1 in fp32; write
// one bf16 result.  Keys are masked by position, so keys past either end of the
// sequence are absent rather than zero (E1), and V rows outside [0, S) are zero
// in LDS so that a zero weight never meets garbage (E2: 0 x NaN = NaN).
//
// Readings this implementation follows (the pages name DyT and lambda but do not
// define them): DyT(x) = gamma[d] tanh(alpha x) + beta[d], one (alpha, gamma,
// beta) set per tensor q1, k1, q2, k2; rotary over all 64 dims, pairs (i, i+32),
// theta_i = p base^(-2i/64), p = token index; o = O_1 - lambda[h] O_2.
//
// The Stable Audio 3 model's own forms (appendix D1, D3, D4, E1), selected per call:
// per-head RMSNorm in place of DyT, x~ = w[d] x / sqrt(mean x^2 + eps); rotary on
// dims 0..31 only (rotate-half pairs i, i+16 at theta_i = p base^(-2i/32), dims
// 32..63 pass through); and V rows of padded tokens taken as zero while their keys
// stay in both softmaxes.  With the 32-dim rotary a thread loads dims (8c, 8c+16)
// for c < 2 and (8c+16, 8c+32) for c >= 2 and stores them where (8c, 8c+32) go
// otherwise: q^ and k^ are held in one common dim order, which leaves q^ . k^ as it is.
//
// Precision plan: DyT, rotation, softmax and subtraction in fp32; the rotated
// q^/k^ (bounded by |gamma| + |beta|) enter Q K^T as fp16 (8x finer than bf16;
// the TPU kernel's bf16 q/k moves near-argmax scores by ~1e-2); P enters P.V as
// bf16 against the bf16 V; rotary angles are reduced in fp64.
//
// Kernels
//   diff_band<NKB>     window <= 8*NKB-8: one workgroup per strip of 64-row blocks
//                      of one (b, h).  The K1/K2/V rows a block can see (its rows
//                      plus a halo on each side) sit prepared in an LDS ring, each
//                      prepared once per strip; each 16-query tile takes all its
//                      in-band keys in one 16*NKB-key slab: one exact softmax per
//                      branch, no rescale.
//   diff_kprep         full (or wide-window) path, pass 1: DyT + rotation of K1 and
//                      K2, once per (b, h) and key -- never once per query block
//                      (V1 / Session 8: re-preparing K per query block was half the
//                      kernel's vector work) -- and V as fp16 (flagged-out rows
//                      zeroed), into the workspace.
//   diff_flash_duo     pass 2: four waves per 32 queries, one branch per wave; q prep
//                      in registers, then a pipelined flash loop over 32-key tiles of the
//                      prepared keys and V; branch 2 is subtracted through LDS at the end.
#include <mutex>
#include <type_traits>
#include <utility>

#include "ka_attn.h"
#include "ka_common.hpp"
#include "ka_kernels.hpp"

namespace ka {

constexpr int KPD = HD + 8;   // LDS pitch of prepared fp16 keys (elements)
constexpr int VPD = HD + 16;  // LDS pitch of V (elements)

struct SharedParams {
  double rev[32];        // revolutions per position, pair i (fp64 angle path)
  float rev_hi[32];      // split fp32 angle path
  float rev_lo[32];
  float gpb[4][HD];      // DyT gamma + beta per set (q1, k1, q2, k2); RMSNorm: the weight
  float m2g[4][HD];      // DyT -2 gamma per set
  float k2a[4];          // 2 log2(e) alpha per set
  float eps;             // RMSNorm
  int split;
};

constexpr int NORM_DYT = 0, NORM_RMS = 1;

template <int NORM>
__device__ __forceinline__ void load_params(SharedParams& sp, const DiffArgs& a) {
  for (int i = threadIdx.x; i < 4 * HD; i += blockDim.x) {
    if constexpr (NORM == NORM_RMS) {
      sp.gpb[i / HD][i % HD] = a.rms_w[i];
    } else {
      const float g = a.gamma[i], b = a.beta[i];
      sp.gpb[i / HD][i % HD] = g + b;
      sp.m2g[i / HD][i % HD] = -2.0f * g;
    }
  }
  if (threadIdx.x < 32) {
    sp.rev[threadIdx.x] = a.rev[threadIdx.x];
    sp.rev_hi[threadIdx.x] = a.rev_hi[threadIdx.x];
    sp.rev_lo[threadIdx.x] = a.rev_lo[threadIdx.x];
  }
  if (NORM == NORM_DYT && threadIdx.x < 4) sp.k2a[threadIdx.x] = 2.0f * LOG2E * a.alpha[threadIdx.x];
  if (threadIdx.x == 0) {
    sp.split = a.split_angles;
    sp.eps = a.rms_eps;
  }
}

// The dims a thread with chunk index c (0..3) holds of a head row: 8 at lo_dim and
// the 8 they pair with (or, past the rotary dims, the next 8 unrotated ones) at
// lo_dim + pair_gap.  Rotary pair index 8c + e in both layouts.
__device__ __forceinline__ int lo_dim(int c, bool rot32) { return rot32 && c >= 2 ? 8 * c + 16 : 8 * c; }
__device__ __forceinline__ int pair_gap(bool rot32) { return rot32 ? 16 : 32; }

// Tensor t (0..5: q1, k1, q2, k2, v, o) of batch element b, head h: the first element of its
// [S][64] slice; token j then sits j * st[t] elements further.
enum { TQ1 = 0, TK1 = 1, TQ2 = 2, TK2 = 3, TV = 4, TO = 5 };
__device__ __forceinline__ size_t slice_at(const DiffArgs& a, int t, size_t b, size_t h) {
  return b * (size_t)a.sb[t] + h * (size_t)a.sh[t];
}
// bytes a buffer resource over one slice spans: S rows at stride st[t], the last one 128 bytes
__device__ __forceinline__ int slice_bytes(const DiffArgs& a, int t) { return ((a.S - 1) * a.st[t] + HD) * 2; }

// Lanes holding one head row: four consecutive lanes (RED_QUAD), eight (RED_OCT) or {l, l^16,
// l^32, l^48} (RED_GROUP4).
constexpr int RED_QUAD = 0, RED_GROUP4 = 1, RED_OCT = 2;
template <int RED>
__device__ __forceinline__ float row_sum(float x) {
  if constexpr (RED == RED_QUAD) return quad_sum(x);
  else if constexpr (RED == RED_OCT) {
    const float y = quad_sum(x);  // then the other quad of the eight (lane ^ 4, swizzle bit mode)
    return y + __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(y), 0x101F));
  } else return group4_sum(x);
}

// The parameters as the preparation reads them: staged in LDS for the whole workgroup ...
struct LdsParamView {
  const SharedParams& sp;
  __device__ bool split() const { return sp.split; }
  __device__ float rev_hi(int i, int) const { return sp.rev_hi[i]; }
  __device__ float rev_lo(int i, int) const { return sp.rev_lo[i]; }
  __device__ double rev(int i, int) const { return sp.rev[i]; }
  __device__ float eps() const { return sp.eps; }
  __device__ float k2a(int t) const { return sp.k2a[t]; }
  __device__ float gpb(int t, int d, int, int) const { return sp.gpb[t][d]; }
  __device__ float m2g(int t, int d, int, int) const { return sp.m2g[t][d]; }
};
// ... or loaded by each thread for its own NP rotary pairs (dims d0 + e and d0 + gap + e) of NSET
// parameter sets straight from global memory (the key-prep pass: k1 and k2; the flash pass: its
// branch's queries): no LDS staging and no barrier before the preparation.
template <int NORM, int NP, int NSET>
struct RegParams {
  float g[NSET][2][NP], b[NSET][2][NP];  // gamma (or the RMS weight) and beta of dims d0 + e, d0 + gap + e
  float rhi[NP], rlo[NP];
  double rv[NP];
  float ka[NSET];
  int t0;  // set of slot 0; slot 1 (when NSET = 2) holds set t0 + 2
  float ep;
  int sp_;
  __device__ RegParams(const DiffArgs& a, int d0, int gap, int i0, int first_set) : t0(first_set) {
    static_assert(NP % 4 == 0, "parameters are read as float4");
#pragma unroll
    for (int s2 = 0; s2 < NSET; ++s2) {
      const int t = first_set + 2 * s2;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int e4 = 0; e4 < NP; e4 += 4) {
          const int d = d0 + hh * gap + e4;
          const float4 gv = *reinterpret_cast<const float4*>((NORM == NORM_RMS ? a.rms_w : a.gamma) + t * HD + d);
          g[s2][hh][e4] = gv.x; g[s2][hh][e4 + 1] = gv.y; g[s2][hh][e4 + 2] = gv.z; g[s2][hh][e4 + 3] = gv.w;
          if constexpr (NORM == NORM_DYT) {
            const float4 bv = *reinterpret_cast<const float4*>(a.beta + t * HD + d);
            b[s2][hh][e4] = bv.x; b[s2][hh][e4 + 1] = bv.y; b[s2][hh][e4 + 2] = bv.z; b[s2][hh][e4 + 3] = bv.w;
          }
        }
      ka[s2] = NORM == NORM_DYT ? 2.0f * LOG2E * a.alpha[t] : 0.0f;
    }
#pragma unroll
    for (int e = 0; e < NP; ++e) {
      rhi[e] = a.rev_hi[i0 + e];
      rlo[e] = a.rev_lo[i0 + e];
      rv[e] = a.rev[i0 + e];
    }
    ep = a.rms_eps;
    sp_ = a.split_angles;
  }
  __device__ int slot(int t) const { return NSET == 1 ? 0 : (t != t0); }
  __device__ bool split() const { return sp_; }
  __device__ float rev_hi(int, int e) const { return rhi[e]; }
  __device__ float rev_lo(int, int e) const { return rlo[e]; }
  __device__ double rev(int, int e) const { return rv[e]; }
  __device__ float eps() const { return ep; }
  __device__ float k2a(int t) const { return ka[slot(t)]; }
  // the values load_params stages: gamma + beta and -2 gamma (DyT), the weight (RMSNorm)
  __device__ float gpb(int t, int, int e, int hh) const {
    return NORM == NORM_RMS ? g[slot(t)][hh][e] : g[slot(t)][hh][e] + b[slot(t)][hh][e];
  }
  __device__ float m2g(int t, int, int e, int hh) const { return -2.0f * g[slot(t)][hh][e]; }
};

// Normalise (DyT, or RMSNorm over the row's 64 dims held by the lanes RED names), then rotate,
// NP rotary pairs (dims d0+e and d0+gap+e, pair index i0+e) of two tensors (parameter sets ta
// and tb) at the same position p; the angles are shared.  ONE: tensor a only.  PV: where the
// parameters come from (LdsParamView or RegParams).
template <int NORM, int RED, bool ONE = false, int NP = 8, class PV>
__device__ __forceinline__ void prep_pairs2(float* alo, float* ahi, float* blo, float* bhi, int d0, int gap, int i0,
                                            int p, int ta, int tb, const PV& sp) {
  const float pf = (float)p;
  // one uniform branch for all the angles, so that the straight-line DyT and rotation
  // below form one block the scheduler can interleave
  float csv[NP], snv[NP];
  if (sp.split()) {
#pragma unroll
    for (int e = 0; e < NP; ++e) rope_cs_split(pf, sp.rev_hi(i0 + e, e), sp.rev_lo(i0 + e, e), csv[e], snv[e]);
  } else {
#pragma unroll
    for (int e = 0; e < NP; ++e) rope_cs_f64(p, sp.rev(i0 + e, e), csv[e], snv[e]);
  }
  float ra = 1.0f, rb = 1.0f;  // RMSNorm: 1 / sqrt(mean x^2 + eps) of each row
  if constexpr (NORM == NORM_RMS) {
    float sa = 0.0f, sb = 0.0f;
#pragma unroll
    for (int e = 0; e < NP; ++e) {
      sa = __builtin_fmaf(alo[e], alo[e], __builtin_fmaf(ahi[e], ahi[e], sa));
      if (!ONE) sb = __builtin_fmaf(blo[e], blo[e], __builtin_fmaf(bhi[e], bhi[e], sb));
    }
    ra = __builtin_amdgcn_rsqf(__builtin_fmaf(row_sum<RED>(sa), 1.0f / HD, sp.eps()));
    if (!ONE) rb = __builtin_amdgcn_rsqf(__builtin_fmaf(row_sum<RED>(sb), 1.0f / HD, sp.eps()));
  }
  const float ka = sp.k2a(ta), kb = sp.k2a(tb);
#pragma unroll
  for (int e = 0; e < NP; ++e) {
    const int dl = d0 + e, dh = d0 + gap + e;
    const float cs = csv[e], sn = snv[e];
    auto norm = [&](float x, int t, int d, int hh, float k, float r) {
      if constexpr (NORM == NORM_RMS) return sp.gpb(t, d, e, hh) * (x * r);
      else return dyt(x, k, sp.gpb(t, d, e, hh), sp.m2g(t, d, e, hh));
    };
    const float a0 = norm(alo[e], ta, dl, 0, ka, ra), a1 = norm(ahi[e], ta, dh, 1, ka, ra);
    // explicit fused forms: every tensor rounds identically, whatever the compiler would contract
    alo[e] = __builtin_fmaf(a0, cs, -(a1 * sn));
    ahi[e] = __builtin_fmaf(a1, cs, a0 * sn);
    if (!ONE) {
      const float b0 = norm(blo[e], tb, dl, 0, kb, rb), b1 = norm(bhi[e], tb, dh, 1, kb, rb);
      blo[e] = __builtin_fmaf(b0, cs, -(b1 * sn));
      bhi[e] = __builtin_fmaf(b1, cs, b0 * sn);
    }
  }
}

// Two fp32 -> two fp16 in one word, rounded toward zero (v_cvt_pkrtz_f16_f32; a value
// representable in fp16 converts exactly either way).
__device__ __forceinline__ unsigned cvt2_f16(float a, float b) {
  return __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_pkrtz(a, b));
}

__device__ __forceinline__ f16x8 cat_f16(i16x4 lo, i16x4 hi) {
  return __builtin_bit_cast(f16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

__device__ __forceinline__ f16x8 to_f16x8(const float* f) {
  f16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (_Float16)pin(f[e]);
  return r;
}
// the same rounding for four values, as their bits
__device__ __forceinline__ uint2 to_f16x4_bits(const float* f) {
  typedef __attribute__((ext_vector_type(4))) _Float16 f16x4;
  f16x4 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) r[e] = (_Float16)pin(f[e]);
  return __builtin_bit_cast(uint2, r);
}

// Load dims [d0, d0+8) and [d0+gap, d0+gap+8) of one bf16 row as fp32 (zeros if !ok).
__device__ __forceinline__ void load_pairs(const unsigned short* row, int d0, int gap, bool ok, float* lo, float* hi) {
  uint4 a = make_uint4(0, 0, 0, 0), b = a;
  if (ok) {
    a = ld16(row + d0);
    b = ld16(row + d0 + gap);
  }
  unpack_bf16x8(a, lo);
  unpack_bf16x8(b, hi);
}

// Workgroups that share a CU are issued oldest first, so with equal work per workgroup the
// youngest one falls behind and finishes alone, on a CU it no longer fills.  A wave that has
// more of its work left takes a higher priority (four levels by the fraction left), so the
// waves of a CU advance together and finish together.
__device__ __forceinline__ void priority_by_work_left(int left, int total) {
  const int lv = (4 * left) / (total + 1);
  if (lv >= 3) __builtin_amdgcn_s_setprio(3);
  else if (lv == 2) __builtin_amdgcn_s_setprio(2);
  else if (lv == 1) __builtin_amdgcn_s_setprio(1);
  else __builtin_amdgcn_s_setprio(0);
}

// ---------------------------------------------------------------- banded, strip-mined
// One workgroup walks a strip of consecutive 64-row blocks of one (b, h).  The
// prepared keys (DyT + rotation, fp16) and the values of every position the
// current block can see -- its rows plus HALO on each side -- live in an LDS ring
// of NR rows; moving to the next block adds 64 new rows and retires 64 old ones,
// so each key is prepared once per strip, not once per block.  The raw rows the
// next block adds, and its queries, are fetched into registers while the current
// block computes.
constexpr int BAND_BM = 64;  // query rows per block step: 4 waves x 16
constexpr int BAND_NW = 4;
#ifndef BAND_TARGET_WGS_SET
#define BAND_TARGET_WGS_SET 768
#endif
constexpr int BAND_TARGET_WGS = BAND_TARGET_WGS_SET;  // about three resident workgroups per CU
#ifndef BAND_WPE
#define BAND_WPE 3
#endif

// One thread's share of one new row: dims [d0, d0+8) and [d0+gap, d0+gap+8) of k1
// and k2 (d0 = lo_dim(cc)), bytes [32cc, 32cc+32) of v, and the row's V flag.
struct RowStage {
  uint4 k1lo, k1hi, k2lo, k2hi, v0, v1;
  unsigned vkeep;
};

// Rows j outside [0, S) read as zero through the buffer resources (a negative row
// offset wraps past the end), so no lane branches.  keep: the V flags of this batch
// index ([S] bytes), read only when the call passes them.
struct BandSrc {
  rsrc_t k1, k2, v, keep;
  int rk1, rk2, rv;  // token strides in bytes
  bool has_keep;
};
__device__ __forceinline__ void stage_load(RowStage& st, const BandSrc& src, int j, int cc, int d0, int gap) {
  const int o1 = j * src.rk1, o2 = j * src.rk2, ov = j * src.rv;
  st.k1lo = buf_ld16(src.k1, o1 + 2 * d0);
  st.k1hi = buf_ld16(src.k1, o1 + 2 * (d0 + gap));
  st.k2lo = buf_ld16(src.k2, o2 + 2 * d0);
  st.k2hi = buf_ld16(src.k2, o2 + 2 * (d0 + gap));
  st.v0 = buf_ld16(src.v, ov + 32 * cc);
  st.v1 = buf_ld16(src.v, ov + 32 * cc + 16);
  // past either end the flag reads 0, and the V row there is zero anyway
  st.vkeep = src.has_keep ? buf_ld1(src.keep, j) : 1u;
}

template <int NORM>
__device__ __forceinline__ void stage_commit(const RowStage& st, unsigned short* K1s, unsigned short* K2s,
                                             unsigned short* Vs, int slot, int j, int cc, int d0, int gap,
                                             bool has_keep, const SharedParams& sp) {
  float k1lo[8], k1hi[8], k2lo[8], k2hi[8];
  unpack_bf16x8(st.k1lo, k1lo);
  unpack_bf16x8(st.k1hi, k1hi);
  unpack_bf16x8(st.k2lo, k2lo);
  unpack_bf16x8(st.k2hi, k2hi);
  // rows no query of the strip sees are prepared too (finite, and masked in every tile)
  prep_pairs2<NORM, RED_QUAD>(k1lo, k1hi, k2lo, k2hi, d0, gap, 8 * cc, j, 1, 3, LdsParamView{sp});
  st16(&K1s[slot * KPD + 8 * cc], __builtin_bit_cast(uint4, to_f16x8(k1lo)));
  st16(&K1s[slot * KPD + 32 + 8 * cc], __builtin_bit_cast(uint4, to_f16x8(k1hi)));
  st16(&K2s[slot * KPD + 8 * cc], __builtin_bit_cast(uint4, to_f16x8(k2lo)));
  st16(&K2s[slot * KPD + 32 + 8 * cc], __builtin_bit_cast(uint4, to_f16x8(k2hi)));
  uint4 v0 = st.v0, v1 = st.v1;
  if (has_keep) {  // uniform; a mask, not a select of two uint4 (which would put the stage in scratch)
    const unsigned m = st.vkeep ? ~0u : 0u;
    v0 = make_uint4(v0.x & m, v0.y & m, v0.z & m, v0.w & m);
    v1 = make_uint4(v1.x & m, v1.y & m, v1.z & m, v1.w & m);
  }
  st16(&Vs[slot * VPD + 16 * cc], v0);
  st16(&Vs[slot * VPD + 16 * cc + 8], v1);
}

// One branch of a 16-query tile against the 16*NKB-key slab starting at ring slot
// s0 (wrapping at NR); exact softmax over the slab; the row sum comes from an
// all-ones MFMA over the same bf16 weights.
template <int NKB, int NR>
__device__ __forceinline__ void band_branch(const unsigned short* Kh, const unsigned short* Vs, int s0,
                                            const f16x8 (&Qf)[2], const bool (&band)[NKB][4], bool edge, int jbase,
                                            int S, float c, int col, int grp, const bf16x8& ones, f32x4 (&O)[4],
                                            float& l) {
  // s0 and NR are multiples of 16, so a ring wrap falls between 16-row groups: the wrapped group
  // start is wave-uniform and the lane adds its row within the group
  f32x4 Sc[NKB];
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
    int sb = s0 + 16 * kb;
    sb = sb >= NR ? sb - NR : sb;
    const unsigned short* kr = Kh + sb * KPD + col * KPD + 8 * grp;
    const f16x8 a0 = *reinterpret_cast<const f16x8*>(kr);
    const f16x8 a1 = *reinterpret_cast<const f16x8*>(kr + 32);
    Sc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, Qf[0], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
    Sc[kb] = mfma_f16(a1, Qf[1], Sc[kb]);
  }
  // the band mask is fixed per lane; keys outside [0, S) occur only in tiles at either end
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int e = 0; e < 4; ++e) Sc[kb][e] = band[kb][e] ? Sc[kb][e] : -INFINITY;
  if (edge) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = jbase + 16 * kb + 4 * grp + e;
        Sc[kb][e] = (j >= 0 && j < S) ? Sc[kb][e] : -INFINITY;
      }
  }
  float mx = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int e = 0; e < 4; ++e) mx = fmaxf(mx, Sc[kb][e]);
  const float mc = group4_max(mx) * c;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int e = 0; e < 4; ++e) Sc[kb][e] = fast_exp2(__builtin_fmaf(Sc[kb][e], c, -mc));
  f32x4 L = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int db = 0; db < 4; ++db) O[db] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < NKB / 2; ++ks) {
    const bf16x8 P = pack_bf16(Sc[2 * ks], Sc[2 * ks + 1]);
    int rb = s0 + 32 * ks;
    rb = rb >= NR ? rb - NR : rb;
    int rb16 = rb + 16;
    rb16 = rb16 >= NR ? rb16 - NR : rb16;
    const int lv = (4 * grp + (col >> 2)) * VPD + 4 * (col & 3);
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const bf16x8 av = cat_bf16(lds_read_tr16(&Vs[rb * VPD + lv + 16 * db]), lds_read_tr16(&Vs[rb16 * VPD + lv + 16 * db]));
      O[db] = mfma_bf16(av, P, O[db]);
    }
    L = mfma_bf16(ones, P, L);
  }
  l = L[0];
}

template <int NKB, int WPE, int NORM>
__global__ __launch_bounds__(64 * BAND_NW) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
void diff_band(DiffArgs a, int nblk, int nstrip) {
  constexpr int HALO = 8 * NKB - 8;       // slab of query tile q0 starts at key q0 - HALO
  constexpr int NR = BAND_BM + 2 * HALO;  // ring rows
  __shared__ __align__(16) unsigned short K1s[NR * KPD];
  __shared__ __align__(16) unsigned short K2s[NR * KPD];
  __shared__ __align__(16) unsigned short Vs[NR * VPD];
  __shared__ SharedParams sp;

  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, grp = lane >> 4, cc = tid & 3;
  const int S = a.S, window = a.window;
  const size_t bh = blockIdx.x / nstrip;  // one-dimensional grid: (b, h) major, strip minor
  const int h = (int)(bh % a.H);
  const size_t bb = bh / a.H;
  const int strip0 = (blockIdx.x % nstrip) * nblk * BAND_BM;
  const int pos0 = strip0 - HALO;  // position held by ring slot 0
  // one (b, h) slice of each tensor; rows outside [0, S) read as zero
  const bool has_keep = a.v_keep != nullptr;
  const BandSrc src{make_rsrc(a.k1 + slice_at(a, TK1, bb, h), slice_bytes(a, TK1)),
                    make_rsrc(a.k2 + slice_at(a, TK2, bb, h), slice_bytes(a, TK2)),
                    make_rsrc(a.v + slice_at(a, TV, bb, h), slice_bytes(a, TV)),
                    make_rsrc(has_keep ? static_cast<const void*>(a.v_keep + bb * (size_t)S) : a.v, S),
                    2 * a.st[TK1], 2 * a.st[TK2], 2 * a.st[TV], has_keep};
  const rsrc_t q1rs = make_rsrc(a.q1 + slice_at(a, TQ1, bb, h), slice_bytes(a, TQ1));
  const rsrc_t q2rs = make_rsrc(a.q2 + slice_at(a, TQ2, bb, h), slice_bytes(a, TQ2));
  const int rq1 = 2 * a.st[TQ1], rq2 = 2 * a.st[TQ2];
  unsigned short* const oslice = a.o + slice_at(a, TO, bb, h);
  const bool rot32 = a.rot32 != 0;
  const int gap = pair_gap(rot32), kd0 = lo_dim(cc, rot32), qd0 = lo_dim(grp, rot32);
  load_params<NORM>(sp, a);
  __syncthreads();

  // fill the ring for the first block: positions pos0 .. pos0 + NR - 1
  for (int r = tid >> 2; r < NR; r += 64 * BAND_NW / 4) {
    const int j = pos0 + r;
    RowStage st;
    stage_load(st, src, j, cc, kd0, gap);
    stage_commit<NORM>(st, K1s, K2s, Vs, r, j, cc, kd0, gap, has_keep, sp);
  }

  // band mask by relative position: key j = q0 - HALO + 16kb + 4grp + e against
  // query p = q0 + col, the same for every tile
  bool band[NKB][4];
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int rel = -HALO + 16 * kb + 4 * grp + e - col;
      band[kb][e] = rel >= -window && rel <= window;
    }
  bf16x8 ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = (__bf16)1.0f;
  const float lam = a.lambda[h];

  // queries of this wave for block 0
  uint4 qs[4];
  auto qload = [&](int r0) {
    const int p = r0 + 16 * w + col;  // rows past S read as zero
    qs[0] = buf_ld16(q1rs, p * rq1 + 2 * qd0);
    qs[1] = buf_ld16(q1rs, p * rq1 + 2 * (qd0 + gap));
    qs[2] = buf_ld16(q2rs, p * rq2 + 2 * qd0);
    qs[3] = buf_ld16(q2rs, p * rq2 + 2 * (qd0 + gap));
  };
  qload(strip0);
  __syncthreads();

  for (int b = 0; b < nblk; ++b) {
    const int r0 = strip0 + b * BAND_BM;
    if (r0 >= S) break;
    priority_by_work_left(nblk - b, nblk);
    const bool more = b + 1 < nblk && r0 + BAND_BM < S;
    // prepared queries of this block
    const int q0 = r0 + 16 * w, p = q0 + col;
    float q1lo[8], q1hi[8], q2lo[8], q2hi[8];
    unpack_bf16x8(qs[0], q1lo);
    unpack_bf16x8(qs[1], q1hi);
    unpack_bf16x8(qs[2], q2lo);
    unpack_bf16x8(qs[3], q2hi);
    prep_pairs2<NORM, RED_GROUP4>(q1lo, q1hi, q2lo, q2hi, qd0, gap, 8 * grp, p, 0, 2, LdsParamView{sp});
    const f16x8 Q1[2] = {to_f16x8(q1lo), to_f16x8(q1hi)};
    const f16x8 Q2[2] = {to_f16x8(q2lo), to_f16x8(q2hi)};
    // fetch what the next block adds while this one computes
    const int jn = r0 + BAND_BM + HALO + (tid >> 2);
    RowStage st;
    if (more) stage_load(st, src, jn, cc, kd0, gap);
    if (more) qload(r0 + BAND_BM);

    const int jbase = q0 - HALO;
    const bool edge = jbase < 0 || jbase + 16 * NKB > S;  // uniform per wave
    const int s0 = (jbase - pos0) % NR;
    f32x4 O1[4], O2[4];
    float l1, l2;
    band_branch<NKB, NR>(K1s, Vs, s0, Q1, band, edge, jbase, S, a.c, col, grp, ones, O1, l1);
    band_branch<NKB, NR>(K2s, Vs, s0, Q2, band, edge, jbase, S, a.c, col, grp, ones, O2, l2);
    {
      // every lane takes part in the store's lane exchange; only rows below S are written
      const float i1 = __builtin_amdgcn_rcpf(l1), i2 = lam * __builtin_amdgcn_rcpf(l2);
      uint2 pk[4];
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        f32x4 r;
#pragma unroll
        for (int e = 0; e < 4; ++e) r[e] = pin(O1[db][e] * i1) - pin(O2[db][e] * i2);
        pk[db] = pack4_bf16_bits(r[0], r[1], r[2], r[3]);
      }
      store_tile_rows(oslice + (size_t)(p < S ? p : 0) * a.st[TO], p < S, grp, pk);
    }
    if (more) {
      __syncthreads();  // every wave is done with the rows about to be replaced
      stage_commit<NORM>(st, K1s, K2s, Vs, (jn - pos0) % NR, jn, cc, kd0, gap, has_keep, sp);
      __syncthreads();
    }
  }
}

// ---------------------------------------------------------------- full path, pass 1: key prep
// Eight threads per key row: lane sub of the octet prepares rotary pairs 4 sub .. 4 sub + 3 of
// both k1 and k2 (their angles computed once for the two tensors) and converts 8 values of V to
// fp16.  Each thread reads its own parameters from global memory, so nothing waits for a
// workgroup barrier.  (Four threads per row holding both tensors left about 1.4 waves per SIMD
// for the 1422-token shape: too few to cover the load and transcendental latencies of this
// short pass.)
template <int NORM>
__global__ __launch_bounds__(256) void diff_kprep(DiffArgs a) {
  const size_t nrows = (size_t)a.B * a.H * a.S;
  const size_t row0 = (size_t)blockIdx.x * 32 + (threadIdx.x >> 3);
  const bool live = row0 < nrows;
  const size_t row = live ? row0 : nrows - 1;  // lanes past the end load a valid row, store nothing
  // lane sub of the octet: rotary pairs 4 sub .. 4 sub + 3 of both k1 and k2 (dims d0 .. d0 + 3 and
  // the four they pair with), so the angles are computed once for the two tensors
  const int sub = threadIdx.x & 7;
  const int j = (int)(row % (size_t)a.S);
  const size_t h = (row / a.S) % a.H, bb = row / a.S / a.H;
  const bool rot32 = a.rot32 != 0;
  const int gap = pair_gap(rot32), d0 = rot32 && sub >= 4 ? 4 * sub + 16 : 4 * sub;
  // the row's loads are issued before the parameter loads, so the two latencies overlap
  const unsigned short* k1r = a.k1 + slice_at(a, TK1, bb, h) + (size_t)j * a.st[TK1];
  const unsigned short* k2r = a.k2 + slice_at(a, TK2, bb, h) + (size_t)j * a.st[TK2];
  const uint2 u1l = ld8(k1r + d0), u1h = ld8(k1r + d0 + gap), u2l = ld8(k2r + d0), u2h = ld8(k2r + d0 + gap);
  // V row: 8 values per thread
  const unsigned short* vr = a.v + slice_at(a, TV, bb, h) + (size_t)j * a.st[TV];
  const uint4 vx = ld16(vr + 8 * sub);
  const bool keep = !a.v_keep || a.v_keep[bb * a.S + j] != 0;
  const RegParams<NORM, 4, 2> prm(a, d0, gap, 4 * sub, 1);  // sets 1 (k1) and 3 (k2)
  if (!live) return;  // whole octets: the lanes of a row leave together
  float alo[4], ahi[4], blo[4], bhi[4];
  unpack_bf16x4(u1l, alo);
  unpack_bf16x4(u1h, ahi);
  unpack_bf16x4(u2l, blo);
  unpack_bf16x4(u2h, bhi);
  prep_pairs2<NORM, RED_OCT, false, 4>(alo, ahi, blo, bhi, d0, gap, 4 * sub, j, 1, 3, prm);
  // the planes hold pair i's rotated dims at i and 32 + i (the layout of the queries' fragments)
  _Float16* w1 = a.ws + row * HD + 4 * sub;
  _Float16* w2 = w1 + nrows * HD;
  st8(w1, to_f16x4_bits(alo));
  st8(w1 + 32, to_f16x4_bits(ahi));
  st8(w2, to_f16x4_bits(blo));
  st8(w2 + 32, to_f16x4_bits(bhi));
  // V as fp16 for pass 2's P.V (exact for 2^-14 <= |v| <= 65504: a bf16 value has 8 significant
  // bits, fp16 11), with the rows of flagged-out tokens zeroed
  const unsigned m = keep ? ~0u : 0u;
  float f[8];
  unpack_bf16x8(make_uint4(vx.x & m, vx.y & m, vx.z & m, vx.w & m), f);
  st16(a.ws + 2 * nrows * HD + row * HD + 8 * sub,
       make_uint4(cvt2_f16(f[0], f[1]), cvt2_f16(f[2], f[3]), cvt2_f16(f[4], f[5]), cvt2_f16(f[6], f[7])));
}

// ---------------------------------------------------------------- full path, pass 2
// The dense kernel's loop on the prepared fp16 keys, one branch per wave: 2 NB waves per
// block, 16 NB queries; waves 0..NB-1 run branch 1 and waves NB..2NB-1 branch 2 for the same
// NB 16-query blocks, so a wave holds one branch's scores, weights and O.  Keys stream in
// 32-key tiles through a two-deep LDS ring (K1 and K2 one tile ahead, V one tile behind);
// step t of a wave
//   * issues the matrix work of S(t+1) = K(t+1) Q^T and of O += V(t-1)^T P(t-1)^T,
//   * forms the weights of tile t on the vector unit, one weight beside each MFMA, the order
//     fixed by scheduling barriers,
//   * requests K1/K2(t+2) and V(t) straight into the ring slots read last before the previous
//     barrier (buffer loads into LDS, no staging registers), waiting for them before its barrier,
// then the block synchronises once.  Weights are 2^(c s - R) with R at the query's running
// maximum (in the exp2 domain), so they stay below 2^F_LAZY until a score passes the maximum
// by F_LAZY: a packed 16-bit maximum over the fp16 weights and a wave-wide vote replace the
// per-tile maximum, and only a voting wave takes maxima and raises R (per query, from its own
// scores).  DyT scores spread widely (a standard deviation near 7 in the exp2 domain): with a
// threshold of 8 a fifth of the wave-steps raise, with 14 about one in thirty; 15 is the largest
// whose weights fp16 still holds (a larger weight converts, toward zero, to 65504, which still
// votes).
// P and V meet as fp16 (the prepared V plane): half the rounding of bf16 weights.  The row sum
// comes from an all-ones MFMA over the same fp16 weights, so O / l is a convex combination.
// At the end branch-2 waves leave lambda O2 / l2 in LDS and branch-1 waves subtract it.
// BAND: keys outside |i - j| <= window are masked and tiles outside the band of the block are
// skipped (windows too wide for the one-pass band kernel).
constexpr int FBN = 32;      // keys per tile
#ifndef F_VSLOT_SET
#define F_VSLOT_SET 1
#endif
#ifndef F_VLEAD_SET
#define F_VLEAD_SET 1
#endif
constexpr int F_VSLOT = F_VSLOT_SET;  // MFMA slot after which a step reads its V fragments
constexpr int F_VLEAD = F_VLEAD_SET;  // vector work runs this many slots ahead of the MFMAs
// One 16-query block per wave (32 queries per workgroup: 720 workgroups for 16 heads x 1422
// tokens, 2.8 per CU) measured faster than two (368 workgroups: 49.5 vs 42.5 us for both passes):
// the finer grid balances the chip better than the longer steps amortise their latency.
#ifndef FULL_NQB
#define FULL_NQB 1
#endif
#ifndef FULL_WPE
#define FULL_WPE 3
#endif
constexpr float R_NONE = -1e30f;  // reference of a query that has seen no key (finite: -inf - -inf = NaN)
constexpr float F_LAZY = 15.0f;   // raise threshold (exp2 domain): weights stay below 2^15
constexpr unsigned short F_VOTE = 0x7800;  // fp16 bit pattern of 2^15

typedef __attribute__((ext_vector_type(2))) unsigned short u16x2;
// Some fp16 half of the four words is >= 2^F_LAZY (non-negative fp16 values order like their
// bit patterns): a packed maximum, then a saturating subtraction of F_VOTE - 1.
__device__ __forceinline__ bool any_f16_at_least_vote(unsigned a, unsigned b, unsigned c, unsigned d) {
  const u16x2 m = __builtin_elementwise_max(
      __builtin_elementwise_max(__builtin_bit_cast(u16x2, a), __builtin_bit_cast(u16x2, b)),
      __builtin_elementwise_max(__builtin_bit_cast(u16x2, c), __builtin_bit_cast(u16x2, d)));
  const u16x2 r = __builtin_elementwise_sub_sat(m, u16x2{(unsigned short)(F_VOTE - 1), (unsigned short)(F_VOTE - 1)});
  return __builtin_bit_cast(unsigned, r) != 0;
}

// Workgroup b of n runs on XCD b % 8: the first 8 floor(n / 8) workgroups are renumbered so that
// XCD x takes a contiguous run of items.
__device__ __forceinline__ int xcd_major(int blk, int n) {
  const int n8 = n & ~7;
  return blk < n8 ? (blk & 7) * (n8 >> 3) + (blk >> 3) : blk;
}

// The rings hold unpadded 128-byte rows whose 16-byte chunks are XOR-swizzled by row, so that the
// fragment reads below hit distinct banks: chunk c of row r sits at chunk position c ^ swz(r).
struct FullLds {
  unsigned short K1[2][FBN * HD];
  unsigned short K2[2][FBN * HD];
  unsigned short V[2][FBN * HD];
};
template <bool BAND, int NORM, int NQB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(FULL_WPE, FULL_WPE)))
void diff_flash_duo(DiffArgs a, int nqb) {
  constexpr int QPW = 16 * NQB;    // queries of a wave
  constexpr int QWG = 2 * QPW;     // queries of a block (two waves per branch)
  static_assert(FBN * 8 == 256, "one 16-byte chunk of each tensor per thread and tile");
  static_assert(2 * 2 * FBN * HD * 2 >= 2 * NQB * 4 * 64 * 16, "the branch-2 hand-over must fit the K rings");
  __shared__ __align__(16) FullLds sm;
  
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const int br = w >> 1;  // 0: branch 1, 1: branch 2 (wave-uniform)
  const int wq = w & 1;   // which half of the block's queries
  const int S = a.S, window = a.window;
  // Workgroups are dispatched round-robin over the 8 XCDs (block b on XCD b % 8), each with its
  // own L2: items are numbered XCD-major, so the blocks of one (b, h) -- which all stream that
  // head's prepared keys and V -- share one L2.
  const int item = xcd_major(blockIdx.x, gridDim.x);
  const size_t bh = item / nqb;  // items: (b, h) major, query block minor
  const int h = (int)(bh % a.H);
  const size_t bb = bh / a.H;
  const size_t base = bh * (size_t)S * HD;  // of the workspace's contiguous planes
  const size_t nrows = (size_t)a.B * a.H * S;
  const bool rot32 = a.rot32 != 0;
  const int gap = pair_gap(rot32), qd0 = lo_dim(grp, rot32);
  const float c = a.c;

  const int qa = (item % nqb) * QWG, qb_ = min(S - 1, qa + QWG - 1);
  const int q0 = qa + QPW * wq;  // first query of this wave; block i holds q0 + 16 i + col

  int t_lo = 0, t_hi = (S - 1) / FBN;
  if (BAND) {
    t_lo = max(0, qa - window) / FBN;
    t_hi = min(S - 1, qb_ + window) / FBN;
  }
  const int T = t_hi - t_lo + 1;
  const int rbytes = S * HD * 2;
  const _Float16* k1h = a.ws + base;
  const _Float16* k2h = a.ws + nrows * HD + base;
  const _Float16* vh = a.ws + 2 * nrows * HD + base;
  // rows past S read as zero through the descriptors
  const u32x4_t k1rs = raw_rsrc(k1h, rbytes), k2rs = raw_rsrc(k2h, rbytes), vrs = raw_rsrc(vh, rbytes);
  // tile u of a tensor into a ring slot: wave w moves rows 8 w .. 8 w + 7 in one instruction, lane l
  // the chunk of row 8 w + l / 8 that belongs at chunk position l % 8
  // The tile offset goes into the descriptor and the ring slot into M0, both scalar; the lane's
  // part of the address is fixed.
  const int drow = 8 * w + (lane >> 3), dpos = lane & 7;
  const int doff_k = drow * (HD * 2) + ((dpos ^ swz_k(drow)) << 4);
  const int doff_v = drow * (HD * 2) + ((dpos ^ swz_v(drow)) << 4);
  constexpr unsigned SLOT = FBN * HD * 2;  // bytes of a ring slot; FullLds holds K1[0..1], K2[0..1], V[0..1]
  static_assert(sizeof(FullLds) == 6 * SLOT, "ring slots are contiguous");
  const unsigned lds_w = lds_addr(&sm.K1[0][0]) + 8 * w * HD * 2;  // this wave's rows in slot 0
  auto dma = [&](const u32x4_t& r, int doff, int u, int slot) {
    load16_to_lds(rsrc_advance(r, (unsigned)(t_lo + u) * SLOT), doff, lds_w + slot * SLOT);
  };
  constexpr int K1S = 0, K2S = 2, VR = 4;  // first slot of each ring
  // the first two key tiles, requested before anything else so that their latency overlaps the
  // query loads and the query preparation
  dma(k1rs, doff_k, 0, K1S);
  dma(k2rs, doff_k, 0, K2S);
  dma(k1rs, doff_k, 1, K1S + 1);  // past the last tile: zeros, never read
  dma(k2rs, doff_k, 1, K2S + 1);
  f16x8 Qf[NQB][2];
  {
    // this branch's queries (q1 with set 0, or q2 with set 2), then the lane's own parameters, both
    // straight from global memory (their latencies overlap, and no barrier precedes the preparation)
    const int tq = br ? TQ2 : TQ1, set = br ? 2 : 0;
    const unsigned short* qt = br ? a.q2 : a.q1;
    float lo[NQB][8], hi[NQB][8];
#pragma unroll
    for (int i = 0; i < NQB; ++i) {
      const int p = q0 + 16 * i + col;
      const size_t pc = p < S ? p : 0;
      load_pairs(qt + slice_at(a, tq, bb, h) + pc * a.st[tq], qd0, gap, p < S, lo[i], hi[i]);
    }
    const RegParams<NORM, 8, 1> prm(a, qd0, gap, 8 * grp, set);
#pragma unroll
    for (int i = 0; i < NQB; ++i) {
      prep_pairs2<NORM, RED_GROUP4, true>(lo[i], hi[i], lo[i], hi[i], qd0, gap, 8 * grp, q0 + 16 * i + col, set, set,
                                          prm);
      Qf[i][0] = to_f16x8(lo[i]);
      Qf[i][1] = to_f16x8(hi[i]);
    }
  }

  const unsigned short(*Kr)[FBN * HD] = br ? sm.K2 : sm.K1;  // this wave's branch keys

  f32x4 O[4][NQB], L[NQB];
  float R[NQB];
  f16x8 P[NQB];
#pragma unroll
  for (int i = 0; i < NQB; ++i) {
    R[i] = R_NONE;
    L[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int db = 0; db < 4; ++db) O[db][i] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  f16x8 ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = (_Float16)1.0f;

  f32x4 Sa[2][NQB], Sb[2][NQB];
  // K fragment (A operand) of 16-key block kb, dims 32 hh + 8 grp .. + 8
  auto kfrag = [&](const unsigned short* Kt, int kb, int hh) {
    const int r = 16 * kb + col;
    return *reinterpret_cast<const f16x8*>(&Kt[r * HD + (((4 * hh + grp) ^ swz_k(r)) << 3)]);
  };
  // V^T fragment (A operand) of dims 16 db .. + 16: lane row = head dim, k = key in the order of the
  // P^T operand (keys 4 grp + e of the first 16-key half, then of the second)
  auto vfrag = [&](const unsigned short* Vt, int db) {
    const int r0 = 4 * grp + (col >> 2), r1 = r0 + 16, ch = 2 * db + ((col & 3) >> 1), half = 4 * (col & 1);
    return cat_f16(lds_read_tr16(&Vt[r0 * HD + ((ch ^ swz_v(r0)) << 3) + half]),
                   lds_read_tr16(&Vt[r1 * HD + ((ch ^ swz_v(r1)) << 3) + half]));
  };
  // prologue: K(0) and K(1) have landed in rings 0 and 1 (a tile past the last is never read); then
  // S(0) = K(0) Q^T
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const f16x8 a0 = kfrag(Kr[0], kb, 0), a1 = kfrag(Kr[0], kb, 1);
#pragma unroll
    for (int i = 0; i < NQB; ++i) {
      Sa[kb][i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, Qf[i][0], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
      Sa[kb][i] = mfma_f16(a1, Qf[i][1], Sa[kb][i]);
    }
  }
  __syncthreads();  // ring 0 is rewritten in step 0

  auto step = [&](auto has_next, auto has_prev, auto parity, int t, f32x4 (&Sc)[2][NQB], f32x4 (&Sn)[2][NQB]) {
    constexpr bool NEXT = decltype(has_next)::value;
    constexpr bool PREV = decltype(has_prev)::value;
    constexpr int PAR = decltype(parity)::value;  // t & 1
    if ((t & 3) == 0) priority_by_work_left(T - t, T);
    // K1 / K2 (t + 2) and V(t) go straight into the ring slots read last before the previous barrier
    // (K(t) for S(t), V(t - 2) for the P.V of step t - 1); they are waited for before this step's
    // barrier
    if (t + 2 < T) {
      dma(k1rs, doff_k, t + 2, K1S + PAR);
      dma(k2rs, doff_k, t + 2, K2S + PAR);
    }
    dma(vrs, doff_v, t, VR + PAR);
    f16x8 kf[2][2], vf[4];
    if (NEXT) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) kf[kb][hh] = kfrag(Kr[PAR ^ 1], kb, hh);
    }
    // V fragments are read right after MFMA slot VS, before the first P.V product (slot NQK);
    // steps without QK work start their P.V products at slot 0 and read them up front
    constexpr int NQK = NEXT ? 4 * NQB : 0;
    constexpr int VS = NEXT ? (F_VSLOT < NQK ? F_VSLOT : NQK - 1) : -1;
    auto load_v = [&]() {
      // V^T A operand: lane row = head dim, k = key in the order of the P^T operand
      const unsigned short* Vt = sm.V[PAR ^ 1];
#pragma unroll
      for (int db = 0; db < 4; ++db) vf[db] = vfrag(Vt, db);
    };
    if (PREV && VS < 0) load_v();
    // keys past S (last tile) or outside the band of some query of the block take no weight
    const int j0 = (t_lo + t) * FBN;
    const bool edge = j0 + FBN > S || (BAND && !(j0 >= qb_ - window && j0 + FBN - 1 <= qa + window));
    if (edge) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = j0 + 16 * kb + 4 * grp + e;
#pragma unroll
          for (int i = 0; i < NQB; ++i) {
            const int p = q0 + 16 * i + col;
            const bool ok = j < S && (!BAND || (j >= p - window && j <= p + window));
            Sc[kb][i][e] = ok ? Sc[kb][i][e] : -INFINITY;
          }
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    constexpr int NM = NQK + (PREV ? 5 * NQB : 0);
    auto mfma_at = [&](auto jj) {
      constexpr int j = decltype(jj)::value;
      if constexpr (j < NQK) {
        constexpr int i = j / 4, kb = (j / 2) % 2, hh = j % 2;
        if constexpr (hh == 0)
          Sn[kb][i] = mfma_f16(kf[kb][0], Qf[i][0], f32x4{0.f, 0.f, 0.f, 0.f});
        else
          Sn[kb][i] = mfma_f16(kf[kb][1], Qf[i][1], Sn[kb][i]);
      } else if constexpr (j < NM) {
        constexpr int jp = j - NQK, i = jp / 5, db = jp % 5;
        if constexpr (db < 4)
          O[db][i] = mfma_f16(vf[db], P[i], O[db][i]);
        else
          L[i] = mfma_f16(ones, P[i], L[i]);
      }
    };
    unsigned Pw[NQB][4];
    float xe[NQB];
    bool vote = false;
    auto valu_at = [&](auto ss) {
      constexpr int sidx = decltype(ss)::value;
      constexpr int i = sidx / 9, e = sidx % 9;
      if constexpr (i < NQB) {
        if constexpr (e < 8) {
          float x = fast_exp2(__builtin_fmaf(Sc[e >> 2][i][e & 3], c, -R[i]));
          asm volatile("" : "+v"(x));  // computed in its slot, not sunk past the next barrier
          if constexpr (e & 1) {
            Pw[i][e >> 1] = cvt2_f16(xe[i], x);
            asm volatile("" : "+v"(Pw[i][e >> 1]));
          } else {
            xe[i] = x;
          }
        } else {
          vote = vote || any_f16_at_least_vote(Pw[i][0], Pw[i][1], Pw[i][2], Pw[i][3]);
        }
      }
    };
    // slot s: MFMA s - F_VLEAD, then vector work s (8 weights per query block, packed in pairs,
    // and the block's vote test)
    constexpr int NSLOT = (NM + F_VLEAD > 9 * NQB) ? NM + F_VLEAD : 9 * NQB;
    [&]<int... SL>(std::integer_sequence<int, SL...>) {
      ([&] {
        constexpr int SM = SL - F_VLEAD;
        if constexpr (SM >= 0) mfma_at(std::integral_constant<int, SM>{});
        if constexpr (PREV && VS >= 0 && SM == VS) load_v();
        valu_at(std::integral_constant<int, SL>{});
        __builtin_amdgcn_sched_barrier(0);
      }(), ...);
    }(std::make_integer_sequence<int, NSLOT>{});
    // some weight of this tile reached 2^F_LAZY, or first tile
    const bool raised = !PREV || __builtin_amdgcn_ballot_w64(vote) != 0;
    if (raised) {
#pragma unroll
      for (int i = 0; i < NQB; ++i) {
        // R moves only for a query whose own largest weight 2^(c max - R) reached 2^F_LAZY (a
        // query that has seen no key keeps R_NONE and weight 0), so a query's result depends on
        // its own scores
        const float lmx = fmaxf(fmaxf(fmaxf(Sc[0][i][0], Sc[0][i][1]), fmaxf(Sc[0][i][2], Sc[0][i][3])),
                                fmaxf(fmaxf(Sc[1][i][0], Sc[1][i][1]), fmaxf(Sc[1][i][2], Sc[1][i][3])));
        const float gmx = group4_max(lmx);
        const float Rn = __builtin_fmaf(gmx, c, -R[i]) >= F_LAZY ? gmx * c : R[i];
        const float alpha = fast_exp2(R[i] - Rn);  // 0 on a query's first keys, 1 where R stays
#pragma unroll
        for (int hh = 0; hh < 4; ++hh)
          Pw[i][hh] = cvt2_f16(fast_exp2(__builtin_fmaf(Sc[hh >> 1][i][2 * (hh & 1)], c, -Rn)),
                               fast_exp2(__builtin_fmaf(Sc[hh >> 1][i][2 * (hh & 1) + 1], c, -Rn)));
        R[i] = Rn;
#pragma unroll
        for (int db = 0; db < 4; ++db) O[db][i] *= alpha;
        L[i] *= alpha;
      }
    }
#pragma unroll
    for (int i = 0; i < NQB; ++i) P[i] = __builtin_bit_cast(f16x8, make_uint4(Pw[i][0], Pw[i][1], Pw[i][2], Pw[i][3]));
    __builtin_amdgcn_s_waitcnt(0);  // this wave's tiles have landed
    __syncthreads();
  };
  using yes = std::integral_constant<bool, true>;
  using no = std::integral_constant<bool, false>;
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  if (T == 1) {
    step(no{}, no{}, P0{}, 0, Sa, Sb);
  } else {
    step(yes{}, no{}, P0{}, 0, Sa, Sb);
    int t = 1;
    for (; t + 2 <= T - 1; t += 2) {
      step(yes{}, yes{}, P1{}, t, Sb, Sa);
      step(yes{}, yes{}, P0{}, t + 1, Sa, Sb);
    }
    if (t < T - 1) {
      step(yes{}, yes{}, P1{}, t, Sb, Sa);
      step(no{}, yes{}, P0{}, t + 1, Sa, Sb);
    } else {
      step(no{}, yes{}, P1{}, t, Sb, Sa);
    }
  }
  {  // P.V of the last tile
    const unsigned short* Vt = sm.V[(T - 1) & 1];
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const f16x8 av = vfrag(Vt, db);
#pragma unroll
      for (int i = 0; i < NQB; ++i) O[db][i] = mfma_f16(av, P[i], O[db][i]);
    }
#pragma unroll
    for (int i = 0; i < NQB; ++i) L[i] = mfma_f16(ones, P[i], L[i]);
  }
  // branch 2 leaves lambda O2 / l2 in LDS (over the K rings, no longer read after the last
  // barrier); branch 1 subtracts it from O1 / l1
  f32x4* X = reinterpret_cast<f32x4*>(&sm.K1[0][0]);  // [2 waves][NQB blocks][4 dim groups][64 lanes]
  const float lam = a.lambda[h];
  if (br) {
#pragma unroll
    for (int i = 0; i < NQB; ++i) {
      const float i2 = lam / L[i][0];
#pragma unroll
      for (int db = 0; db < 4; ++db)
        X[((wq * NQB + i) * 4 + db) * 64 + lane] = f32x4{pin(O[db][i][0] * i2), pin(O[db][i][1] * i2),
                                                         pin(O[db][i][2] * i2), pin(O[db][i][3] * i2)};
    }
  }
  __syncthreads();
  if (!br) {
#pragma unroll
    for (int i = 0; i < NQB; ++i) {
      const int p = q0 + 16 * i + col;
      // every lane takes part in the store's lane exchange; only rows below S are written
      const float i1 = 1.0f / L[i][0];
      uint2 pk[4];
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const f32x4 x = X[((wq * NQB + i) * 4 + db) * 64 + lane];
        f32x4 r;
#pragma unroll
        for (int e = 0; e < 4; ++e) r[e] = pin(O[db][i][e] * i1) - x[e];
        pk[db] = pack4_bf16_bits(r[0], r[1], r[2], r[3]);
      }
      store_tile_rows(a.o + slice_at(a, TO, bb, h) + (size_t)(p < S ? p : 0) * a.st[TO], p < S, grp, pk);
    }
  }
}

// ---------------------------------------------------------------- dispatch
static bool use_band(int S, int window) { return window >= 0 && window < S - 1 && window <= BAND_MAX_WINDOW; }

// full path: k1^, k2^ and V (with flagged rows zeroed), all fp16
size_t diff_workspace_bytes(int B, int H, int S, int window, bool v_flags) {
  (void)v_flags;
  if (use_band(S, window)) return 0;
  return (size_t)3 * B * H * S * HD * sizeof(_Float16);
}

// ---------------------------------------------------------------- allocation-free workspace
// One copy per GPU of a file-scope device array, for callers that cannot allocate (stream
// capture, serving loops).  On the host the array's name only stands in for the symbol: its
// device address comes from hipGetSymbolAddress, looked up once per device with that device
// current, and only that address is ever passed to a kernel.  The array keeps the last
// call's contents; the full path overwrites every byte it reads (prepared keys) before
// reading it, so nothing is cleared.  Calls that overlap on one GPU share it and race.
__device__ __align__(256) unsigned char scratch[KA_STATIC_WORKSPACE_BYTES];

hipError_t diff_static_workspace(void** ptr, size_t* bytes) {
  static std::mutex mu;
  static void* addr[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  *bytes = KA_STATIC_WORKSPACE_BYTES;
  return hipSuccess;
}

hipError_t launch_diffattn(const DiffArgs& a0, hipStream_t s) {
  DiffArgs a = a0;
  if (a.window >= a.S - 1) a.window = -1;  // the band covers every key: full attention
  const int BH = a.B * a.H;
  if (use_band(a.S, a.window)) {
    // strips of nblk consecutive 64-row blocks, about BAND_TARGET_WGS workgroups in all
    const int nb = (a.S + BAND_BM - 1) / BAND_BM;
    int nblk = (int)(((long long)nb * BH + BAND_TARGET_WGS - 1) / BAND_TARGET_WGS);
    nblk = nblk < 1 ? 1 : (nblk > 16 ? 16 : nblk);
    const int nstrip = (nb + nblk - 1) / nblk;
    const dim3 grid(nstrip * BH);
    const bool narrow = a.window <= 24;
    if (a.norm == NORM_RMS) {
      if (narrow)
        hipLaunchKernelGGL((diff_band<4, BAND_WPE, NORM_RMS>), grid, dim3(64 * BAND_NW), 0, s, a, nblk, nstrip);
      else
        hipLaunchKernelGGL((diff_band<6, 2, NORM_RMS>), grid, dim3(64 * BAND_NW), 0, s, a, nblk, nstrip);
    } else {
      if (narrow)
        hipLaunchKernelGGL((diff_band<4, BAND_WPE, NORM_DYT>), grid, dim3(64 * BAND_NW), 0, s, a, nblk, nstrip);
      else
        hipLaunchKernelGGL((diff_band<6, 2, NORM_DYT>), grid, dim3(64 * BAND_NW), 0, s, a, nblk, nstrip);
    }
    return hipGetLastError();
  }
  const size_t nrows = (size_t)BH * a.S;
  const dim3 kgrid((unsigned)((nrows + 31) / 32));
  if (a.norm == NORM_RMS)
    hipLaunchKernelGGL(diff_kprep<NORM_RMS>, kgrid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(diff_kprep<NORM_DYT>, kgrid, dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  constexpr int NQB = FULL_NQB, QWG = 32 * NQB;  // query blocks per wave, queries per workgroup
  const int nqb = (a.S + QWG - 1) / QWG;
  const dim3 grid(nqb * BH);
  if (a.norm == NORM_RMS) {
    if (a.window >= 0)
      hipLaunchKernelGGL((diff_flash_duo<true, NORM_RMS, NQB>), grid, dim3(256), 0, s, a, nqb);
    else
      hipLaunchKernelGGL((diff_flash_duo<false, NORM_RMS, NQB>), grid, dim3(256), 0, s, a, nqb);
  } else {
    if (a.window >= 0)
      hipLaunchKernelGGL((diff_flash_duo<true, NORM_DYT, NQB>), grid, dim3(256), 0, s, a, nqb);
    else
      hipLaunchKernelGGL((diff_flash_duo<false, NORM_DYT, NQB>), grid, dim3(256), 0, s, a, nqb);
  }
  return hipGetLastError();
}

}  // namespace ka
