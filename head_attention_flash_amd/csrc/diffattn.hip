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
//                      kernel's vector work) -- into the fp16 workspace.
//   diff_flash<..>     pass 2: q prep in registers, then a two-branch flash loop
//                      over 64-key tiles of the prepared keys and V.
#include "ka_common.hpp"
#include "ka_kernels.hpp"

namespace ka {

constexpr int KPD = HD + 8;   // LDS pitch of prepared fp16 keys (elements)
constexpr int VPD = HD + 16;  // LDS pitch of V (elements)

struct SharedParams {
  double rev[32];        // revolutions per position, pair i (fp64 angle path)
  float rev_hi[32];      // split fp32 angle path
  float rev_lo[32];
  float gpb[4][HD];      // DyT gamma + beta per set (q1, k1, q2, k2)
  float m2g[4][HD];      // DyT -2 gamma per set
  float k2a[4];          // 2 log2(e) alpha per set
  int split;
};

__device__ __forceinline__ void load_params(SharedParams& sp, const DiffArgs& a) {
  for (int i = threadIdx.x; i < 4 * HD; i += blockDim.x) {
    const float g = a.gamma[i], b = a.beta[i];
    sp.gpb[i / HD][i % HD] = g + b;
    sp.m2g[i / HD][i % HD] = -2.0f * g;
  }
  if (threadIdx.x < 32) {
    sp.rev[threadIdx.x] = a.rev[threadIdx.x];
    sp.rev_hi[threadIdx.x] = a.rev_hi[threadIdx.x];
    sp.rev_lo[threadIdx.x] = a.rev_lo[threadIdx.x];
  }
  if (threadIdx.x < 4) sp.k2a[threadIdx.x] = 2.0f * LOG2E * a.alpha[threadIdx.x];
  if (threadIdx.x == 0) sp.split = a.split_angles;
}

// DyT then rotation, for 8 rotary pairs (dims i0+e and i0+32+e) of two tensors
// (parameter sets ta and tb) at the same position p; the angles are shared.
__device__ __forceinline__ void prep_pairs2(float* alo, float* ahi, float* blo, float* bhi, int i0, int p, int ta,
                                            int tb, const SharedParams& sp) {
  const float ka = sp.k2a[ta], kb = sp.k2a[tb];
  const float pf = (float)p;
  const bool split = sp.split;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int i = i0 + e;
    float cs, sn;
    if (split)
      rope_cs_split(pf, sp.rev_hi[i], sp.rev_lo[i], cs, sn);
    else
      rope_cs_f64(p, sp.rev[i], cs, sn);
    const float a0 = dyt(alo[e], ka, sp.gpb[ta][i], sp.m2g[ta][i]);
    const float a1 = dyt(ahi[e], ka, sp.gpb[ta][i + 32], sp.m2g[ta][i + 32]);
    // explicit fused forms: every tensor rounds identically, whatever the compiler would contract
    alo[e] = __builtin_fmaf(a0, cs, -(a1 * sn));
    ahi[e] = __builtin_fmaf(a1, cs, a0 * sn);
    const float b0 = dyt(blo[e], kb, sp.gpb[tb][i], sp.m2g[tb][i]);
    const float b1 = dyt(bhi[e], kb, sp.gpb[tb][i + 32], sp.m2g[tb][i + 32]);
    blo[e] = __builtin_fmaf(b0, cs, -(b1 * sn));
    bhi[e] = __builtin_fmaf(b1, cs, b0 * sn);
  }
}

__device__ __forceinline__ f16x8 to_f16x8(const float* f) {
  f16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (_Float16)pin(f[e]);
  return r;
}

// Load dims [i0, i0+8) and [i0+32, i0+40) of one bf16 row as fp32 (zeros if !ok).
__device__ __forceinline__ void load_pairs(const unsigned short* row, int i0, bool ok, float* lo, float* hi) {
  uint4 a = make_uint4(0, 0, 0, 0), b = a;
  if (ok) {
    a = ld16(row + i0);
    b = ld16(row + i0 + 32);
  }
  unpack_bf16x8(a, lo);
  unpack_bf16x8(b, hi);
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
constexpr int BAND_TARGET_WGS = 768;  // about three resident workgroups per CU
#ifndef BAND_WPE
#define BAND_WPE 3
#endif

// One thread's share of one new row: dims [8cc, 8cc+8) and [8cc+32, 8cc+40) of k1
// and k2, and bytes [32cc, 32cc+32) of v.
struct RowStage {
  uint4 k1lo, k1hi, k2lo, k2hi, v0, v1;
};

__device__ __forceinline__ void stage_load(RowStage& st, const DiffArgs& a, size_t base, int j, bool ok, int cc) {
  st.k1lo = st.k1hi = st.k2lo = st.k2hi = st.v0 = st.v1 = make_uint4(0, 0, 0, 0);
  if (ok) {
    const size_t off = base + (size_t)j * HD;
    st.k1lo = ld16(a.k1 + off + 8 * cc);
    st.k1hi = ld16(a.k1 + off + 32 + 8 * cc);
    st.k2lo = ld16(a.k2 + off + 8 * cc);
    st.k2hi = ld16(a.k2 + off + 32 + 8 * cc);
    st.v0 = ld16(a.v + off + 16 * cc);
    st.v1 = ld16(a.v + off + 16 * cc + 8);
  }
}

__device__ __forceinline__ void stage_commit(const RowStage& st, unsigned short* K1s, unsigned short* K2s,
                                             unsigned short* Vs, int slot, int j, bool ok, int cc,
                                             const SharedParams& sp) {
  float k1lo[8], k1hi[8], k2lo[8], k2hi[8];
  unpack_bf16x8(st.k1lo, k1lo);
  unpack_bf16x8(st.k1hi, k1hi);
  unpack_bf16x8(st.k2lo, k2lo);
  unpack_bf16x8(st.k2hi, k2hi);
  if (ok) prep_pairs2(k1lo, k1hi, k2lo, k2hi, 8 * cc, j, 1, 3, sp);  // rows outside stay zero
  st16(&K1s[slot * KPD + 8 * cc], __builtin_bit_cast(uint4, to_f16x8(k1lo)));
  st16(&K1s[slot * KPD + 32 + 8 * cc], __builtin_bit_cast(uint4, to_f16x8(k1hi)));
  st16(&K2s[slot * KPD + 8 * cc], __builtin_bit_cast(uint4, to_f16x8(k2lo)));
  st16(&K2s[slot * KPD + 32 + 8 * cc], __builtin_bit_cast(uint4, to_f16x8(k2hi)));
  st16(&Vs[slot * VPD + 16 * cc], st.v0);
  st16(&Vs[slot * VPD + 16 * cc + 8], st.v1);
}

// One branch of a 16-query tile against the 16*NKB-key slab starting at ring slot
// s0 (wrapping at NR); exact softmax over the slab; the row sum comes from an
// all-ones MFMA over the same bf16 weights.
template <int NKB, int NR>
__device__ __forceinline__ void band_branch(const unsigned short* Kh, const unsigned short* Vs, int s0,
                                            const f16x8 (&Qf)[2], const bool (&ok)[NKB][4], float c, int col,
                                            int grp, const bf16x8& ones, f32x4 (&O)[4], float& l) {
  f32x4 Sc[NKB];
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
    int s = s0 + 16 * kb + col;
    s = s >= NR ? s - NR : s;
    const f16x8 a0 = *reinterpret_cast<const f16x8*>(&Kh[s * KPD + 8 * grp]);
    const f16x8 a1 = *reinterpret_cast<const f16x8*>(&Kh[s * KPD + 32 + 8 * grp]);
    Sc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, Qf[0], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
    Sc[kb] = mfma_f16(a1, Qf[1], Sc[kb]);
  }
  float mx = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      Sc[kb][e] = ok[kb][e] ? Sc[kb][e] : -INFINITY;
      mx = fmaxf(mx, Sc[kb][e]);
    }
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
    int r = s0 + 32 * ks + 4 * grp + (col >> 2);
    r = r >= NR ? r - NR : r;
    int r16 = r + 16;
    r16 = r16 >= NR ? r16 - NR : r16;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int vcol = 16 * db + 4 * (col & 3);
      const bf16x8 av = cat_bf16(lds_read_tr16(&Vs[r * VPD + vcol]), lds_read_tr16(&Vs[r16 * VPD + vcol]));
      O[db] = mfma_bf16(av, P, O[db]);
    }
    L = mfma_bf16(ones, P, L);
  }
  l = L[0];
}

template <int NKB, int WPE>
__global__ __launch_bounds__(64 * BAND_NW) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
void diff_band(DiffArgs a, int nblk) {
  constexpr int HALO = 8 * NKB - 8;       // slab of query tile q0 starts at key q0 - HALO
  constexpr int NR = BAND_BM + 2 * HALO;  // ring rows
  __shared__ __align__(16) unsigned short K1s[NR * KPD];
  __shared__ __align__(16) unsigned short K2s[NR * KPD];
  __shared__ __align__(16) unsigned short Vs[NR * VPD];
  __shared__ SharedParams sp;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int col = lane & 15, grp = lane >> 4, cc = tid & 3;
  const int S = a.S, window = a.window;
  const size_t bh = blockIdx.y;
  const int h = (int)(bh % a.H);
  const size_t base = bh * (size_t)S * HD;
  const int strip0 = blockIdx.x * nblk * BAND_BM;
  const int pos0 = strip0 - HALO;  // position held by ring slot 0
  // every key any query of the strip can see; other rows are kept zero (and masked)
  const int send = min(S, strip0 + nblk * BAND_BM);
  const int jlo = max(0, strip0 - window), jhi = min(S - 1, send - 1 + window);
  load_params(sp, a);
  __syncthreads();

  // fill the ring for the first block: positions pos0 .. pos0 + NR - 1
  for (int r = tid >> 2; r < NR; r += 64 * BAND_NW / 4) {
    const int j = pos0 + r;
    const bool ok = j >= jlo && j <= jhi;
    RowStage st;
    stage_load(st, a, base, j, ok, cc);
    stage_commit(st, K1s, K2s, Vs, r, j, ok, cc, sp);
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
    const int p = r0 + 16 * w + col;
    qs[0] = qs[1] = qs[2] = qs[3] = make_uint4(0, 0, 0, 0);
    if (p < S) {
      const size_t off = base + (size_t)p * HD;
      qs[0] = ld16(a.q1 + off + 8 * grp);
      qs[1] = ld16(a.q1 + off + 32 + 8 * grp);
      qs[2] = ld16(a.q2 + off + 8 * grp);
      qs[3] = ld16(a.q2 + off + 32 + 8 * grp);
    }
  };
  qload(strip0);
  __syncthreads();

  for (int b = 0; b < nblk; ++b) {
    const int r0 = strip0 + b * BAND_BM;
    if (r0 >= S) break;
    const bool more = b + 1 < nblk && r0 + BAND_BM < S;
    // prepared queries of this block
    const int q0 = r0 + 16 * w, p = q0 + col;
    float q1lo[8], q1hi[8], q2lo[8], q2hi[8];
    unpack_bf16x8(qs[0], q1lo);
    unpack_bf16x8(qs[1], q1hi);
    unpack_bf16x8(qs[2], q2lo);
    unpack_bf16x8(qs[3], q2hi);
    prep_pairs2(q1lo, q1hi, q2lo, q2hi, 8 * grp, p, 0, 2, sp);
    const f16x8 Q1[2] = {to_f16x8(q1lo), to_f16x8(q1hi)};
    const f16x8 Q2[2] = {to_f16x8(q2lo), to_f16x8(q2hi)};
    // fetch what the next block adds while this one computes
    const int jn = r0 + BAND_BM + HALO + (tid >> 2);
    const bool okn = more && jn >= jlo && jn <= jhi;
    RowStage st;
    stage_load(st, a, base, jn, okn, cc);
    if (more) qload(r0 + BAND_BM);

    const int jbase = q0 - HALO;
    bool ok[NKB][4];
    const bool edge = jbase < 0 || jbase + 16 * NKB > S;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = jbase + 16 * kb + 4 * grp + e;
        ok[kb][e] = band[kb][e] && (!edge || (j >= 0 && j < S));
      }
    const int s0 = (jbase - pos0) % NR;
    f32x4 O1[4], O2[4];
    float l1, l2;
    band_branch<NKB, NR>(K1s, Vs, s0, Q1, ok, a.c, col, grp, ones, O1, l1);
    band_branch<NKB, NR>(K2s, Vs, s0, Q2, ok, a.c, col, grp, ones, O2, l2);
    if (p < S) {
      const float i1 = 1.0f / l1, i2 = lam / l2;
      unsigned short* orow = a.o + base + (size_t)p * HD;
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        f32x4 r;
#pragma unroll
        for (int e = 0; e < 4; ++e) r[e] = pin(O1[db][e] * i1) - pin(O2[db][e] * i2);
        st8(orow + 16 * db + 4 * grp, pack4_bf16_bits(r[0], r[1], r[2], r[3]));
      }
    }
    if (more) {
      __syncthreads();  // every wave is done with the rows about to be replaced
      stage_commit(st, K1s, K2s, Vs, (jn - pos0) % NR, jn, okn, cc, sp);
      __syncthreads();
    }
  }
}

// ---------------------------------------------------------------- full path, pass 1: key prep
__global__ __launch_bounds__(256) void diff_kprep(DiffArgs a) {
  __shared__ SharedParams sp;
  load_params(sp, a);
  __syncthreads();
  const size_t nrows = (size_t)a.B * a.H * a.S;
  const size_t row = (size_t)blockIdx.x * 64 + (threadIdx.x >> 2);
  const int cc = threadIdx.x & 3;
  if (row >= nrows) return;
  const int j = (int)(row % (size_t)a.S);
  float k1lo[8], k1hi[8], k2lo[8], k2hi[8];
  load_pairs(a.k1 + row * HD, 8 * cc, true, k1lo, k1hi);
  load_pairs(a.k2 + row * HD, 8 * cc, true, k2lo, k2hi);
  prep_pairs2(k1lo, k1hi, k2lo, k2hi, 8 * cc, j, 1, 3, sp);
  _Float16* w1 = a.ws + row * HD;
  _Float16* w2 = a.ws + nrows * HD + row * HD;
  st16(w1 + 8 * cc, __builtin_bit_cast(uint4, to_f16x8(k1lo)));
  st16(w1 + 32 + 8 * cc, __builtin_bit_cast(uint4, to_f16x8(k1hi)));
  st16(w2 + 8 * cc, __builtin_bit_cast(uint4, to_f16x8(k2lo)));
  st16(w2 + 32 + 8 * cc, __builtin_bit_cast(uint4, to_f16x8(k2hi)));
}

// ---------------------------------------------------------------- full path, pass 2: two-branch flash
constexpr int DBN = 64;  // keys per tile

template <int NQB>
__device__ __forceinline__ void flash_branch_tile(const unsigned short* Kt, const unsigned short* Vt,
                                                  const f16x8 (&Qf)[NQB][2], int j0, int q0, int window, int S,
                                                  float c, int col, int grp, float (&m)[NQB], float (&l)[NQB],
                                                  f32x4 (&O)[4][NQB]) {
  f32x4 Sc[4][NQB];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
    for (int i = 0; i < NQB; ++i) Sc[kb][i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const f16x8 a = *reinterpret_cast<const f16x8*>(&Kt[(16 * kb + col) * KPD + 32 * t + 8 * grp]);
#pragma unroll
      for (int i = 0; i < NQB; ++i) Sc[kb][i] = mfma_f16(a, Qf[i][t], Sc[kb][i]);
    }
  }
  const bool need_mask = (j0 + DBN > S) || (window >= 0);
  if (need_mask) {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = j0 + 16 * kb + 4 * grp + e;
#pragma unroll
        for (int i = 0; i < NQB; ++i) {
          const int p = q0 + 16 * i + col;
          const bool ok = (j < S) && (window < 0 || (j >= p - window && j <= p + window));
          Sc[kb][i][e] = ok ? Sc[kb][i][e] : -INFINITY;
        }
      }
  }
#pragma unroll
  for (int i = 0; i < NQB; ++i) {
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int e = 0; e < 4; ++e) mx = fmaxf(mx, Sc[kb][i][e]);
    mx = group4_max(mx);
    const float mnew = fmaxf(m[i], mx);
    // a row that has seen no key yet (possible under a band) keeps m = -inf, l = 0, O = 0
    const bool none = mnew == -INFINITY;
    const float alpha = none ? 1.0f : fast_exp2((m[i] - mnew) * c);
    const float mc = none ? 0.0f : mnew * c;
    m[i] = mnew;
    float ls = 0.0f;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float pv = fast_exp2(__builtin_fmaf(Sc[kb][i][e], c, -mc));
        Sc[kb][i][e] = pv;
        ls += pv;
      }
    l[i] = __builtin_fmaf(l[i], alpha, ls);
#pragma unroll
    for (int db = 0; db < 4; ++db) O[db][i] *= alpha;
  }
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    bf16x8 P[NQB];
#pragma unroll
    for (int i = 0; i < NQB; ++i) P[i] = pack_bf16(Sc[2 * ks][i], Sc[2 * ks + 1][i]);
    const int vrow = 32 * ks + 4 * grp + (col >> 2);
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int vcol = 16 * db + 4 * (col & 3);
      const bf16x8 av = cat_bf16(lds_read_tr16(&Vt[vrow * VPD + vcol]), lds_read_tr16(&Vt[(vrow + 16) * VPD + vcol]));
#pragma unroll
      for (int i = 0; i < NQB; ++i) O[db][i] = mfma_bf16(av, P[i], O[db][i]);
    }
  }
}

template <int NQB, int NW>
__global__ __launch_bounds__(64 * NW) void diff_flash(DiffArgs a) {
  __shared__ __align__(16) unsigned short K1s[2][DBN * KPD];
  __shared__ __align__(16) unsigned short K2s[2][DBN * KPD];
  __shared__ __align__(16) unsigned short Vs[2][DBN * VPD];
  __shared__ SharedParams sp;
  constexpr int NT = 64 * NW;
  constexpr int CPT = DBN * 8 / NT;
  static_assert(CPT * NT == DBN * 8, "tile must split evenly over the block");

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int S = a.S, window = a.window;
  const size_t bh = blockIdx.y;
  const int h = (int)(bh % a.H);
  const size_t base = bh * (size_t)S * HD;
  const size_t nrows = (size_t)a.B * a.H * S;
  const unsigned short* k1h = reinterpret_cast<const unsigned short*>(a.ws) + base;
  const unsigned short* k2h = reinterpret_cast<const unsigned short*>(a.ws) + nrows * HD + base;
  const unsigned short* vb = a.v + base;
  load_params(sp, a);
  __syncthreads();

  const int qblk0 = blockIdx.x * NW * 16 * NQB;  // first query of the workgroup
  const int q0 = qblk0 + w * 16 * NQB;           // first query of this wave
  f16x8 Q1[NQB][2], Q2[NQB][2];
#pragma unroll
  for (int i = 0; i < NQB; ++i) {
    const int p = q0 + 16 * i + col;
    float q1lo[8], q1hi[8], q2lo[8], q2hi[8];
    const size_t po = p < S ? (size_t)p * HD : 0;
    load_pairs(a.q1 + base + po, 8 * grp, p < S, q1lo, q1hi);
    load_pairs(a.q2 + base + po, 8 * grp, p < S, q2lo, q2hi);
    prep_pairs2(q1lo, q1hi, q2lo, q2hi, 8 * grp, p, 0, 2, sp);
    Q1[i][0] = to_f16x8(q1lo);
    Q1[i][1] = to_f16x8(q1hi);
    Q2[i][0] = to_f16x8(q2lo);
    Q2[i][1] = to_f16x8(q2hi);
  }

  // key tiles this workgroup can see
  int t_lo = 0, t_hi = (S - 1) / DBN;
  if (window >= 0) {
    const int qlast = min(S - 1, qblk0 + NW * 16 * NQB - 1);
    t_lo = max(0, qblk0 - window) / DBN;
    t_hi = min(S - 1, qlast + window) / DBN;
  }

  f32x4 O1[4][NQB], O2[4][NQB];
  float m1[NQB], l1[NQB], m2[NQB], l2[NQB];
#pragma unroll
  for (int i = 0; i < NQB; ++i) {
    m1[i] = m2[i] = -INFINITY;
    l1[i] = l2[i] = 0.0f;
#pragma unroll
    for (int db = 0; db < 4; ++db) O1[db][i] = O2[db][i] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  uint4 r1[CPT], r2[CPT], rv[CPT];
  auto gload = [&](int tile) {
#pragma unroll
    for (int ch = 0; ch < CPT; ++ch) {
      const int idx = tid + ch * NT, r = idx >> 3, cc = idx & 7;
      const int j = tile * DBN + r;
      r1[ch] = r2[ch] = rv[ch] = make_uint4(0, 0, 0, 0);
      if (j < S) {
        r1[ch] = ld16(k1h + (size_t)j * HD + cc * 8);
        r2[ch] = ld16(k2h + (size_t)j * HD + cc * 8);
        rv[ch] = ld16(vb + (size_t)j * HD + cc * 8);
      }
    }
  };
  auto swrite = [&](int buf) {
#pragma unroll
    for (int ch = 0; ch < CPT; ++ch) {
      const int idx = tid + ch * NT, r = idx >> 3, cc = idx & 7;
      st16(&K1s[buf][r * KPD + cc * 8], r1[ch]);
      st16(&K2s[buf][r * KPD + cc * 8], r2[ch]);
      st16(&Vs[buf][r * VPD + cc * 8], rv[ch]);
    }
  };

  gload(t_lo);
  swrite(0);
  __syncthreads();
  for (int t = t_lo; t <= t_hi; ++t) {
    const int buf = (t - t_lo) & 1;
    if (t < t_hi) gload(t + 1);
    flash_branch_tile<NQB>(K1s[buf], Vs[buf], Q1, t * DBN, q0, window, S, a.c, col, grp, m1, l1, O1);
    flash_branch_tile<NQB>(K2s[buf], Vs[buf], Q2, t * DBN, q0, window, S, a.c, col, grp, m2, l2, O2);
    if (t < t_hi) swrite(buf ^ 1);
    __syncthreads();
  }

  const float lam = a.lambda[h];
#pragma unroll
  for (int i = 0; i < NQB; ++i) {
    const int p = q0 + 16 * i + col;
    const float i1 = 1.0f / group4_sum(l1[i]);
    const float i2 = lam / group4_sum(l2[i]);
    if (p < S) {
      unsigned short* orow = a.o + base + (size_t)p * HD;
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        f32x4 r;
#pragma unroll
        for (int e = 0; e < 4; ++e) r[e] = pin(O1[db][i][e] * i1) - pin(O2[db][i][e] * i2);
        st8(orow + 16 * db + 4 * grp, pack4_bf16_bits(r[0], r[1], r[2], r[3]));
      }
    }
  }
}

// ---------------------------------------------------------------- dispatch
static bool use_band(int S, int window) { return window >= 0 && window < S - 1 && window <= BAND_MAX_WINDOW; }

size_t diff_workspace_bytes(int B, int H, int S, int window) {
  if (use_band(S, window)) return 0;
  return (size_t)2 * B * H * S * HD * sizeof(_Float16);
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
    dim3 grid((nb + nblk - 1) / nblk, BH);
    if (a.window <= 24)
      hipLaunchKernelGGL((diff_band<4, BAND_WPE>), grid, dim3(64 * BAND_NW), 0, s, a, nblk);
    else
      hipLaunchKernelGGL((diff_band<6, 2>), grid, dim3(64 * BAND_NW), 0, s, a, nblk);
    return hipGetLastError();
  }
  const size_t nrows = (size_t)BH * a.S;
  hipLaunchKernelGGL(diff_kprep, dim3((unsigned)((nrows + 63) / 64)), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  constexpr int NQB = 1, NW = 4;
  dim3 grid((a.S + 16 * NQB * NW - 1) / (16 * NQB * NW), BH);
  hipLaunchKernelGGL((diff_flash<NQB, NW>), grid, dim3(64 * NW), 0, s, a);
  return hipGetLastError();
}

}  // namespace ka
