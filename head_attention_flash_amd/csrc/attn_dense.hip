// attn_dense.hip -- dense and cross scaled-dot-product attention for gfx950.
//
// Definition ("SDXL as a requirements inventory", s1.3, CrossAttention): per
// (b, h, i), o = sum_j softmax_j(scale <q_i, k_j>) v_j over all Sk keys, no mask.
// The score matrix is never materialised (s2.4 of the same page: level-1
// self-attention scores would be 335 MB per image); keys stream through an
// online softmax (running max and sum, the accumulator rescaled per key tile),
// which reaches the two-pass softmax result in exact arithmetic.
//
// Kernels
//   attn_f32_kernel        fp32 in/out, fp32 arithmetic; one thread per query.
//   attn_bf16_duo<NA, NB>  bf16 in/out, the large-grid path: 8 waves per block, two
//                          per SIMD, each owning NA (waves 0-3) or NB (waves 4-7)
//                          16-query blocks; S^T = K Q^T and O^T = V^T P^T on
//                          v_mfma_f32_16x16x32_bf16 with fp32 softmax; 32-key K/V
//                          tiles double-buffered in LDS; the matrix instructions of
//                          one tile are interleaved by hand with the exponentials of
//                          the previous one.  The 1/sum is applied once per output
//                          row after P.V (the "divide after P.V" trim of "401 -> 163
//                          ms: Stable Audio 3 medium on one TPU v6e chip", s4).
//   attn_bf16_pipe<..>     the same arithmetic with 16 queries per wave and 64-key
//                          tiles, four waves per SIMD: grids too small to fill the
//                          chip with the 8-wave blocks.
//   xattn_bf16<..>         cross-attention for short key sets: every key and value
//                          of a (b, h) is loaded into LDS once and re-read by every
//                          query tile ("SDXL as a requirements inventory" s5.7: hold
//                          the re-read operand, stream Q/O); one exact softmax pass.
//
// Softmax bookkeeping shared by the bf16 kernels:
//   * the row sum comes from the matrix core: one extra MFMA per 32 keys multiplies
//     P^T by an all-ones A operand, so the sum is taken over the same bf16-rounded
//     weights that meet V, with no VALU add per score;
//   * the running maximum is raised lazily (LAZY_LOG2 in ka_common.hpp).
// This file is compiled without NaN semantics (-fno-honor-nans): the maxima are
// taken on finite scores or -inf, and IEEE NaN quieting would double their cost.
#include <algorithm>
#include <atomic>
#include <type_traits>
#include <utility>

#include "ka_common.hpp"
#include "ka_kernels.hpp"

namespace ka {

// ---------------------------------------------------------------- fp32
constexpr int F32_BQ = 128;  // queries per block (one per thread)
constexpr int F32_BK = 32;   // keys per LDS tile

__global__ __launch_bounds__(F32_BQ) void attn_f32_kernel(const float* __restrict__ q, const float* __restrict__ k,
                                                          const float* __restrict__ v, float* __restrict__ o, int Sq,
                                                          int Sk, float scale, int nqb) {
  __shared__ __align__(16) float ks[F32_BK][HD];
  __shared__ __align__(16) float vs[F32_BK][HD];
  const int tid = threadIdx.x;
  const size_t bh = blockIdx.x / nqb;  // one-dimensional grid: (b, h) major, query block minor
  const int i = (blockIdx.x % nqb) * F32_BQ + tid;
  const float* qb = q + bh * (size_t)Sq * HD;
  const float* kb = k + bh * (size_t)Sk * HD;
  const float* vb = v + bh * (size_t)Sk * HD;

  float qr[HD], acc[HD];
#pragma unroll
  for (int d = 0; d < HD; ++d) {
    qr[d] = (i < Sq) ? qb[(size_t)i * HD + d] : 0.0f;
    acc[d] = 0.0f;
  }
  float m = -INFINITY, l = 0.0f;
  for (int j0 = 0; j0 < Sk; j0 += F32_BK) {
    __syncthreads();
    for (int idx = tid; idx < F32_BK * (HD / 4); idx += F32_BQ) {
      const int r = idx / (HD / 4), c = (idx % (HD / 4)) * 4;
      float4 kk = make_float4(0.f, 0.f, 0.f, 0.f), vv = kk;
      if (j0 + r < Sk) {
        kk = *reinterpret_cast<const float4*>(kb + (size_t)(j0 + r) * HD + c);
        vv = *reinterpret_cast<const float4*>(vb + (size_t)(j0 + r) * HD + c);
      }
      *reinterpret_cast<float4*>(&ks[r][c]) = kk;
      *reinterpret_cast<float4*>(&vs[r][c]) = vv;
    }
    __syncthreads();
    const int nk = min(F32_BK, Sk - j0);
    float s[F32_BK];
    float mt = m;
#pragma unroll
    for (int jj = 0; jj < F32_BK; ++jj) {
      float dot = 0.0f;
#pragma unroll
      for (int d = 0; d < HD; ++d) dot = __builtin_fmaf(qr[d], ks[jj][d], dot);
      s[jj] = dot * scale;
      if (jj < nk) mt = fmaxf(mt, s[jj]);
    }
    const float alpha = expf(m - mt);  // m = -inf on the first tile: alpha = 0
    l *= alpha;
#pragma unroll
    for (int d = 0; d < HD; ++d) acc[d] *= alpha;
#pragma unroll
    for (int jj = 0; jj < F32_BK; ++jj) {
      const float p = (jj < nk) ? expf(s[jj] - mt) : 0.0f;
      l += p;
#pragma unroll
      for (int d = 0; d < HD; ++d) acc[d] = __builtin_fmaf(p, vs[jj][d], acc[d]);
    }
    m = mt;
  }
  if (i < Sq) {
    const float inv = 1.0f / l;
    float* ob = o + bh * (size_t)Sq * HD + (size_t)i * HD;
#pragma unroll
    for (int d = 0; d < HD; d += 4)
      *reinterpret_cast<float4*>(ob + d) = make_float4(acc[d] * inv, acc[d + 1] * inv, acc[d + 2] * inv, acc[d + 3] * inv);
  }
}

// ---------------------------------------------------------------- bf16 constants
// LDS pitches (in 16-bit elements): K rows are read as 16-byte A-operand chunks,
// V rows through the transposed 8-byte read; both pitches keep a wave's reads on
// distinct banks.
#ifndef DENSE_KPAD
#define DENSE_KPAD 8
#endif
#ifndef DENSE_VPAD
#define DENSE_VPAD 16
#endif
constexpr int KP = HD + DENSE_KPAD;
constexpr int VP = HD + DENSE_VPAD;
constexpr int BN = 64;  // keys per tile of the 16-query kernel

// ---------------------------------------------------------------- bf16, 16 queries per wave, software-pipelined
// The matrix core and the vector unit work at the same time inside one wave:
// while the softmax of key tile t runs on the VALU, the wave has already issued
// the MFMAs of S(t+1) = K(t+1) Q^T and of O += V(t-1)^T P(t-1)^T, which do not
// depend on it.  LDS holds K one tile ahead and V one tile behind:
//   iteration t reads  Kb[(t+1)&1] = K(t+1) and Vb[(t-1)&1] = V(t-1),
//   and writes         Kb[t&1] <- K(t+2),   Vb[t&1] <- V(t),
// buffers last read in iteration t-1, so one barrier per iteration suffices.
template <int NQB>
struct PipeRegs {
  f32x4 O[4][NQB];
  f32x4 L[NQB];
  float m[NQB];
  bf16x8 P[2][NQB];  // weights of the previous tile, consumed by its P.V
};

template <int NQB>
__device__ __forceinline__ void pipe_qk(const unsigned short* Kt, const bf16x8 (&Qf)[NQB][2], int col, int grp,
                                        f32x4 (&S)[4][NQB]) {
#pragma unroll
  for (int kb4 = 0; kb4 < 4; ++kb4) {
    const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(&Kt[(16 * kb4 + col) * KP + 8 * grp]);
    const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(&Kt[(16 * kb4 + col) * KP + 32 + 8 * grp]);
#pragma unroll
    for (int i = 0; i < NQB; ++i) {
      // first half of the head dim starts from a zero accumulator (inline constant)
      S[kb4][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, Qf[i][0], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
      S[kb4][i] = mfma_bf16(a1, Qf[i][1], S[kb4][i]);
    }
  }
}

template <int NQB>
__device__ __forceinline__ void pipe_pv(const unsigned short* Vt, const bf16x8& ones, int col, int grp,
                                        PipeRegs<NQB>& R) {
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const int vrow = 32 * ks + 4 * grp + (col >> 2);
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int vcol = 16 * db + 4 * (col & 3);
      const bf16x8 a = cat_bf16(lds_read_tr16(&Vt[vrow * VP + vcol]), lds_read_tr16(&Vt[(vrow + 16) * VP + vcol]));
#pragma unroll
      for (int i = 0; i < NQB; ++i) R.O[db][i] = mfma_bf16(a, R.P[ks][i], R.O[db][i]);
    }
#pragma unroll
    for (int i = 0; i < NQB; ++i) R.L[i] = mfma_bf16(ones, R.P[ks][i], R.L[i]);
  }
}

// Softmax of one tile (weights against the lazily raised maximum) into R.P; returns
// per q-block whether the maximum was raised, with the rescale factor in alpha.
template <int NQB, bool MASK>
__device__ __forceinline__ bool pipe_softmax(f32x4 (&S)[4][NQB], int j0, int Sk, float c, int grp,
                                             PipeRegs<NQB>& R, float (&alpha)[NQB]) {
  if (MASK) {
#pragma unroll
    for (int kb4 = 0; kb4 < 4; ++kb4)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool ok = j0 + 16 * kb4 + 4 * grp + e < Sk;
#pragma unroll
        for (int i = 0; i < NQB; ++i) S[kb4][i][e] = ok ? S[kb4][i][e] : -INFINITY;
      }
  }
  bool any = false;
#pragma unroll
  for (int i = 0; i < NQB; ++i) {
    float mx = S[0][i][0];
#pragma unroll
    for (int kb4 = 0; kb4 < 4; ++kb4)
#pragma unroll
      for (int e = 0; e < 4; ++e) mx = fmaxf(mx, S[kb4][i][e]);
    mx = group4_max(mx);
    const bool raise = (mx - R.m[i]) * c > LAZY_LOG2;  // true on the first tile (m = -inf)
    const float mnew = raise ? mx : R.m[i];
    alpha[i] = fast_exp2((R.m[i] - mnew) * c);        // 1 when not raised; no branch
    R.m[i] = mnew;
    any = any || raise;
    const float mc = mnew * c;
#pragma unroll
    for (int kb4 = 0; kb4 < 4; ++kb4)
#pragma unroll
      for (int e = 0; e < 4; ++e) S[kb4][i][e] = fast_exp2(__builtin_fmaf(S[kb4][i][e], c, -mc));
  }
  return any;
}

template <int NQB>
__device__ __forceinline__ void pipe_pack(const f32x4 (&S)[4][NQB], PipeRegs<NQB>& R) {
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int i = 0; i < NQB; ++i) {
      R.P[ks][i] = pack_bf16(S[2 * ks][i], S[2 * ks + 1][i]);
      // materialise the weights here, inside the region where they overlap the
      // matrix work, rather than letting them sink past the rescale branch
      asm volatile("" : "+v"(R.P[ks][i]));
    }
}

template <int NQB>
__device__ __forceinline__ void pipe_rescale(bool any, const float (&alpha)[NQB], PipeRegs<NQB>& R) {
  if (__builtin_amdgcn_ballot_w64(any)) {
#pragma unroll
    for (int i = 0; i < NQB; ++i) {
#pragma unroll
      for (int db = 0; db < 4; ++db) R.O[db][i] *= alpha[i];
      R.L[i] *= alpha[i];
    }
  }
}

// IL > 0: ask the scheduler to interleave each MFMA with IL vector instructions.
template <int NQB, int NW, int IL, int WPE = 0>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(WPE > 0 ? WPE : 1, WPE > 0 ? WPE : 8)))
void attn_bf16_pipe(const unsigned short* __restrict__ q,
                                                          const unsigned short* __restrict__ k,
                                                          const unsigned short* __restrict__ v,
                                                          unsigned short* __restrict__ o, int Sq, int Sk, float c,
                                                          int nbh) {
  __shared__ __align__(16) unsigned short Kb[2][BN * KP];
  __shared__ __align__(16) unsigned short Vb[2][BN * VP];
  constexpr int NT = 64 * NW;
  constexpr int CPT = (BN * 8 + NT - 1) / NT;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int col = lane & 15, grp = lane >> 4;
  // Workgroups are dispatched round-robin over the 8 XCDs, each with its own L2.
  // Renumber them so that every XCD works through a contiguous run of (b, h, query
  // block) items: the blocks of one (b, h) then share that XCD's L2 copy of K and V.
  const int nqb = gridDim.x / nbh;  // query blocks per (b, h); the grid is nqb * nbh
  const int nwg = gridDim.x, nwg8 = nwg & ~7;
  int item = blockIdx.x;
  if (item < nwg8) item = (item & 7) * (nwg8 >> 3) + (item >> 3);
  const size_t bh = item / nqb;
  const int q0 = ((item % nqb) * NW + w) * (16 * NQB);
  const unsigned short* qb = q + bh * (size_t)Sq * HD;
  const unsigned short* kbase = k + bh * (size_t)Sk * HD;
  const unsigned short* vbase = v + bh * (size_t)Sk * HD;

  bf16x8 Qf[NQB][2];
#pragma unroll
  for (int i = 0; i < NQB; ++i) {
    const int row = q0 + 16 * i + col;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      uint4 u = make_uint4(0, 0, 0, 0);
      if (row < Sq) u = ld16(qb + (size_t)row * HD + 32 * t + 8 * grp);
      Qf[i][t] = __builtin_bit_cast(bf16x8, u);
    }
  }
  PipeRegs<NQB> R;
#pragma unroll
  for (int i = 0; i < NQB; ++i) {
    R.m[i] = -INFINITY;
    R.L[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int db = 0; db < 4; ++db) R.O[db][i] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  bf16x8 ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = (__bf16)1.0f;

  const int T = (Sk + BN - 1) / BN;
  // K and V of this (b, h) as buffer resources: rows past Sk read as zero
  const rsrc_t krs = make_rsrc(kbase, Sk * HD * 2);
  const rsrc_t vrs = make_rsrc(vbase, Sk * HD * 2);
  uint4 kr[CPT], vr[CPT];
  auto gload = [&](const rsrc_t& src, int tile, uint4 (&r)[CPT]) {
#pragma unroll
    for (int ch = 0; ch < CPT; ++ch) {
      const int idx = tid + ch * NT;
      r[ch] = buf_ld16(src, tile * (BN * HD * 2) + idx * 16);
    }
  };
  auto swrite = [&](unsigned short* dst, int pitch, const uint4 (&r)[CPT]) {
#pragma unroll
    for (int ch = 0; ch < CPT; ++ch) {
      const int idx = tid + ch * NT, rr = idx >> 3, cc = idx & 7;
      if (CPT * NT == BN * 8 || idx < BN * 8) st16(&dst[rr * pitch + cc * 8], r[ch]);
    }
  };

  // prologue: S(0) from K(0); K(1) into the other buffer
  f32x4 Sa[4][NQB], Sb[4][NQB];
  gload(krs, 0, kr);
  swrite(Kb[0], KP, kr);
  __syncthreads();
  pipe_qk<NQB>(Kb[0], Qf, col, grp, Sa);
  if (T > 1) {
    gload(krs, 1, kr);
    swrite(Kb[1], KP, kr);
  }
  __syncthreads();

  // one pipelined iteration t: S_next = K(t+1) Q^T and P.V of tile t-1 on the matrix
  // core, softmax of tile t (in S_cur) on the vector unit
  auto step = [&](auto has_next, auto has_prev, int t, f32x4 (&Scur)[4][NQB], f32x4 (&Snext)[4][NQB]) {
    constexpr bool NEXT = decltype(has_next)::value;
    constexpr bool PREV = decltype(has_prev)::value;
    if (NEXT) gload(krs, t + 2, kr);  // past the last tile: zeros, never written
    gload(vrs, t, vr);
    if (NEXT) pipe_qk<NQB>(Kb[(t + 1) & 1], Qf, col, grp, Snext);
    if (PREV) pipe_pv<NQB>(Vb[(t - 1) & 1], ones, col, grp, R);
    float alpha[NQB];
    const bool any = NEXT ? pipe_softmax<NQB, false>(Scur, t * BN, Sk, c, grp, R, alpha)
                          : pipe_softmax<NQB, true>(Scur, t * BN, Sk, c, grp, R, alpha);
    if (IL > 0) {
      // matrix work of this region: 16*NQB MFMAs for S(t+1), 18*NQB for P.V(t-1)
      constexpr int NM = (NEXT ? 8 * NQB : 0) + (PREV ? 10 * NQB : 0);
#pragma unroll
      for (int i = 0; i < NM; ++i) {
        __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 1, 0);
        __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
        __builtin_amdgcn_sched_group_barrier(SG_VALU, IL, 0);
      }
    }
    pipe_pack<NQB>(Scur, R);
    pipe_rescale<NQB>(any, alpha, R);
    if (NEXT && t + 2 < T) swrite(Kb[t & 1], KP, kr);
    swrite(Vb[t & 1], VP, vr);
    __syncthreads();
  };
  using yes = std::integral_constant<bool, true>;
  using no = std::integral_constant<bool, false>;

  if (T == 1) {
    step(no{}, no{}, 0, Sa, Sb);
  } else {
    step(yes{}, no{}, 0, Sa, Sb);
    int t = 1;
    for (; t + 2 <= T - 1; t += 2) {
      step(yes{}, yes{}, t, Sb, Sa);
      step(yes{}, yes{}, t + 1, Sa, Sb);
    }
    if (t < T - 1) {
      step(yes{}, yes{}, t, Sb, Sa);
      step(no{}, yes{}, t + 1, Sa, Sb);
    } else {
      step(no{}, yes{}, t, Sb, Sa);
    }
  }
  pipe_pv<NQB>(Vb[(T - 1) & 1], ones, col, grp, R);

  unsigned short* ob = o + bh * (size_t)Sq * HD;
#pragma unroll
  for (int i = 0; i < NQB; ++i) {
    const float inv = 1.0f / R.L[i][0];
    const int row = q0 + 16 * i + col;
    uint2 pk[4];
#pragma unroll
    for (int db = 0; db < 4; ++db)
      pk[db] = pack4_bf16_bits(R.O[db][i][0] * inv, R.O[db][i][1] * inv, R.O[db][i][2] * inv, R.O[db][i][3] * inv);
    store_tile_rows(ob + (size_t)(row < Sq ? row : 0) * HD, row < Sq, grp, pk);
  }
}

// ---------------------------------------------------------------- bf16, 8 waves per block
// Block layout: 512 threads, two waves per SIMD.  Waves 0-3 own NA query blocks of
// 16 queries each, waves 4-7 own NB, so one SIMD carries NA + NB blocks and a block
// covers 64 (NA + NB) queries of one (b, h).  Keys stream in 32-key tiles through a
// two-deep LDS ring; step t of a wave
//   * issues the matrix work of S(t+1) = K(t+1) Q^T and of O += V(t-1)^T P(t-1)^T,
//   * computes the weights of tile t on the vector unit, one weight (or one bf16
//     pack) beside each MFMA, the instruction order fixed by scheduling barriers,
//   * requests K(t+2) / V(t) straight into the ring slots read last before the previous
//     barrier (buffer loads into LDS: no staging registers, no LDS stores; each wave moves
//     8 rows of a tile and waits for them right before the barrier),
// then the block synchronises once.  Waves 0-3 move K, waves 4-7 move V.
//
// Vector work is what bounds this loop on CDNA4 (an MFMA hides little of it), so a
// weight takes one FMA and one v_exp and nothing else but the bf16 pack:
//   * the weight is 2^(c*s - R), c = scale * log2(e) applied to the fp32 score (Q as
//     given: a bf16 rounding of c*q would move scores by up to 2^-9 of sum |c q_d k_d|);
//   * R sits LAZY_LOG2 - 1 above the running maximum, so every weight stays below 2
//     unless a score passes the maximum by LAZY_LOG2.  Weights >= 2 are the bf16 values
//     with bit 14 set: one OR over the packed weights and a wave-wide vote replace the
//     per-tile maximum.  Only on a vote (and on the first tile) are the four-lane maxima
//     taken, R raised, this tile's weights recomputed, and O, l rescaled.
// The common 2^-(LAZY_LOG2 - 1) factor of the weights cancels in O / l.
constexpr int DBN = 32;       // keys per tile
constexpr int DUO_VSLOT = 5;  // MFMA slot at which a step reads its V fragments
constexpr int DUO_VLEAD = 1;  // vector work runs this many slots ahead of the MFMAs

// unpadded 128-byte rows, 16-byte chunks XOR-swizzled by row (swz_k, swz_v)
struct DuoLds {
  unsigned short K[2][DBN * HD];
  unsigned short V[2][DBN * HD];
};

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
__device__ __forceinline__ unsigned cvt2_bf16(float a, float b) {
  bf16x2 v;
  v[0] = (__bf16)a;
  v[1] = (__bf16)b;
  return __builtin_bit_cast(unsigned, v);
}

// QUAD = false: 512-thread block, waves 0-3 move the K tiles and waves 4-7 the V tiles.  QUAD =
// true: 256-thread block, every wave moves 8 rows of each K and V tile.
template <int NQB, bool QUAD>
__device__ __forceinline__ void duo_wave(DuoLds& sm, const unsigned short* __restrict__ qb, int Sq, int q0,
                                         const unsigned short* kbase, const unsigned short* vbase, int Sk, float c,
                                         unsigned short* __restrict__ ob, int tid) {
  const int lane = tid & 63, col = lane & 15, grp = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool isK = QUAD || w < 4;  // the 8-wave form: waves 0-3 move K, 4-7 move V
  // rows past Sk read as zero through the descriptors
  const u32x4_t krs = raw_rsrc(kbase, Sk * HD * 2), vrs = raw_rsrc(vbase, Sk * HD * 2);
  // a tile into a ring slot: wave w (of the four that move a tensor) moves rows 8 (w % 4) .. + 7 in
  // one instruction, lane l the chunk of row 8 (w % 4) + l / 8 that belongs at chunk position l % 8
  const int wl = w & 3, drow = 8 * wl + (lane >> 3), dpos = lane & 7;
  const int doff_k = drow * (HD * 2) + ((dpos ^ swz_k(drow)) << 4);
  const int doff_v = drow * (HD * 2) + ((dpos ^ swz_v(drow)) << 4);
  // the tile offset goes into the descriptor and the ring slot into M0, both scalar
  constexpr unsigned SLOT = DBN * HD * 2;  // bytes of a ring slot
  const unsigned lds_k = lds_addr(&sm.K[0][8 * wl * HD]), lds_v = lds_addr(&sm.V[0][8 * wl * HD]);
  auto dma_k = [&](int tile, int slot) {
    load16_to_lds(rsrc_advance(krs, (unsigned)tile * SLOT), doff_k, lds_k + slot * SLOT);
  };
  auto dma_v = [&](int tile, int slot) {
    load16_to_lds(rsrc_advance(vrs, (unsigned)tile * SLOT), doff_v, lds_v + slot * SLOT);
  };
  // K fragment (A operand) of 16-key block kb, dims 32 h + 8 grp .. + 8
  auto kfrag = [&](const unsigned short* Kt, int kb, int h) {
    const int r = 16 * kb + col;
    return *reinterpret_cast<const bf16x8*>(&Kt[r * HD + (((4 * h + grp) ^ swz_k(r)) << 3)]);
  };
  // V^T fragment (A operand) of dims 16 db .. + 16: lane row = head dim, k = key in the order of the
  // P^T operand (keys 4 grp + e of the first 16-key half, then of the second)
  auto vfrag = [&](const unsigned short* Vt, int db) {
    const int r0 = 4 * grp + (col >> 2), r1 = r0 + 16, ch = 2 * db + ((col & 3) >> 1), half = 4 * (col & 1);
    return cat_bf16(lds_read_tr16(&Vt[r0 * HD + ((ch ^ swz_v(r0)) << 3) + half]),
                    lds_read_tr16(&Vt[r1 * HD + ((ch ^ swz_v(r1)) << 3) + half]));
  };

  bf16x8 Qf[NQB][2];
#pragma unroll
  for (int i = 0; i < NQB; ++i) {
    const int row = q0 + 16 * i + col;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      uint4 u = make_uint4(0, 0, 0, 0);
      if (row < Sq) u = ld16(qb + (size_t)row * HD + 32 * t + 8 * grp);
      Qf[i][t] = __builtin_bit_cast(bf16x8, u);  // as given: c is applied to each score in fp32
    }
  }
  f32x4 O[4][NQB], L[NQB];
  // R: exp2-domain reference, LAZY_LOG2 - 1 above the running maximum; the weights 2^(c*s - R) stay
  // below 2 until some score passes the maximum by LAZY_LOG2: then (and on the first tile) R is raised.
  float R[NQB];
  bf16x8 P[NQB];
#pragma unroll
  for (int i = 0; i < NQB; ++i) {
    R[i] = -INFINITY;
    L[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int db = 0; db < 4; ++db) O[db][i] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  bf16x8 ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = (__bf16)1.0f;

  const int T = (Sk + DBN - 1) / DBN;
  f32x4 Sa[2][NQB], Sb[2][NQB];
  // prologue: K(0) -> K[0] and K(1) -> K[1] (a tile past the last is never read), then S(0) = K(0) Q^T
  if (isK) {
    dma_k(0, 0);
    dma_k(1, 1);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const bf16x8 a0 = kfrag(sm.K[0], kb, 0), a1 = kfrag(sm.K[0], kb, 1);
#pragma unroll
    for (int i = 0; i < NQB; ++i) {
      Sa[kb][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, Qf[i][0], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
      Sa[kb][i] = mfma_bf16(a1, Qf[i][1], Sa[kb][i]);
    }
  }
  __syncthreads();  // K[0] is rewritten in step 0

  auto step = [&](auto has_next, auto has_prev, auto parity, int t, f32x4 (&Sc)[2][NQB], f32x4 (&Sn)[2][NQB]) {
    constexpr bool NEXT = decltype(has_next)::value;
    constexpr bool PREV = decltype(has_prev)::value;
    constexpr int PAR = decltype(parity)::value;  // t & 1
    // K(t+2) and V(t) go straight into the ring slots read last before the previous barrier (K(t) for
    // S(t), V(t-2) for the P.V of step t-1); each wave waits for its own before this step's barrier
    if (isK && t + 2 < T) dma_k(t + 2, PAR);
    if (QUAD || !isK) dma_v(t, PAR);
    bf16x8 kf[2][2], vf[4];
    if (NEXT) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int h = 0; h < 2; ++h) kf[kb][h] = kfrag(sm.K[PAR ^ 1], kb, h);
    }
    // V fragments are read at MFMA slot DUO_VSLOT, after the K fragments have been consumed by the first
    // QK products; steps without QK work start their P.V products at slot 0 and read them up front
    constexpr int VS = NEXT ? (DUO_VSLOT < 4 * NQB ? DUO_VSLOT : 4 * NQB - 1) : -1;  // before the first P.V
    auto load_v = [&]() {
      // V^T A operand: lane row = head dim, k = key in the order of the P^T operand
      // (keys 4*grp + e of the first 16-key half, then of the second)
      const unsigned short* Vt = sm.V[PAR ^ 1];
#pragma unroll
      for (int db = 0; db < 4; ++db) vf[db] = vfrag(Vt, db);
    };
    if (PREV && VS < 0) load_v();
    if (!NEXT) {  // last tile: keys past Sk take no weight
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool ok = t * DBN + 16 * kb + 4 * grp + e < Sk;
#pragma unroll
          for (int i = 0; i < NQB; ++i) Sc[kb][i][e] = ok ? Sc[kb][i][e] : -INFINITY;
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    constexpr int NQK = NEXT ? 4 * NQB : 0;
    constexpr int NM = NQK + (PREV ? 5 * NQB : 0);
    auto mfma_at = [&](auto jj) {
      constexpr int j = decltype(jj)::value;
      if constexpr (j < NQK) {
        constexpr int i = j / 4, kb = (j / 2) % 2, h = j % 2;
        if constexpr (h == 0)
          Sn[kb][i] = mfma_bf16(kf[kb][0], Qf[i][0], f32x4{0.f, 0.f, 0.f, 0.f});
        else
          Sn[kb][i] = mfma_bf16(kf[kb][1], Qf[i][1], Sn[kb][i]);
      } else if constexpr (j < NM) {
        constexpr int jp = j - NQK, i = jp / 5, db = jp % 5;
        if constexpr (db < 4)
          O[db][i] = mfma_bf16(vf[db], P[i], O[db][i]);
        else
          L[i] = mfma_bf16(ones, P[i], L[i]);
      }
    };
    unsigned Pw[NQB][4];
    float xe[NQB];
    unsigned orb[NQB];
    auto valu_at = [&](auto ss) {
      constexpr int s = decltype(ss)::value;
      constexpr int i = s / 9, e = s % 9;
      if constexpr (i < NQB) {
        if constexpr (e < 8) {
          float x = fast_exp2(__builtin_fmaf(Sc[e >> 2][i][e & 3], c, -R[i]));
          asm volatile("" : "+v"(x));  // computed in its slot, not sunk past the next barrier
          if constexpr (e & 1) {
            Pw[i][e >> 1] = cvt2_bf16(xe[i], x);
            asm volatile("" : "+v"(Pw[i][e >> 1]));
          } else {
            xe[i] = x;
          }
        } else {
          orb[i] = Pw[i][0] | Pw[i][1] | Pw[i][2] | Pw[i][3];
        }
      }
    };
    // slot s: MFMA s - DUO_VLEAD, then vector work s (8 weights, packed in pairs, and one OR per query
    // block): the first slots hold only weights, which need no LDS data, while the K fragments arrive
    constexpr int NSLOT = (NM + DUO_VLEAD > 9 * NQB) ? NM + DUO_VLEAD : 9 * NQB;
    [&]<int... S>(std::integer_sequence<int, S...>) {
      ([&] {
        constexpr int SM = S - DUO_VLEAD;
        if constexpr (SM >= 0) mfma_at(std::integral_constant<int, SM>{});
        if constexpr (PREV && VS >= 0 && SM == VS) load_v();
        valu_at(std::integral_constant<int, S>{});
        __builtin_amdgcn_sched_barrier(0);
      }(), ...);
    }(std::make_integer_sequence<int, NSLOT>{});
    // some weight of this tile reached 2 (bit 14 of a bf16 half), or first tile
    unsigned orall = 0;
#pragma unroll
    for (int i = 0; i < NQB; ++i) orall |= orb[i];
    const bool raised = !PREV || __builtin_amdgcn_ballot_w64((orall & 0x40004000u) != 0) != 0;
    if (raised) {
#pragma unroll
      for (int i = 0; i < NQB; ++i) {
        // R moves only for a query whose own largest weight, 2^(c max - R), reached 2 (always on
        // the first tile, where R = -inf), so a query's result never depends on the other queries
        // of its wave; every such query is in a wave that voted
        const float lmx = fmaxf(fmaxf(fmaxf(Sc[0][i][0], Sc[0][i][1]), fmaxf(Sc[0][i][2], Sc[0][i][3])),
                                fmaxf(fmaxf(Sc[1][i][0], Sc[1][i][1]), fmaxf(Sc[1][i][2], Sc[1][i][3])));
        const float gmx = group4_max(lmx);
        const float Rn = __builtin_fmaf(gmx, c, -R[i]) >= 1.0f ? __builtin_fmaf(gmx, c, LAZY_LOG2 - 1.f) : R[i];
        const float alpha = fast_exp2(R[i] - Rn);  // 0 on the first tile, 1 where R stays
#pragma unroll
        for (int h = 0; h < 4; ++h)
          Pw[i][h] = cvt2_bf16(fast_exp2(__builtin_fmaf(Sc[h >> 1][i][2 * (h & 1)], c, -Rn)),
                               fast_exp2(__builtin_fmaf(Sc[h >> 1][i][2 * (h & 1) + 1], c, -Rn)));
        R[i] = Rn;
#pragma unroll
        for (int db = 0; db < 4; ++db) O[db][i] *= alpha;
        L[i] *= alpha;
      }
    }
#pragma unroll
    for (int i = 0; i < NQB; ++i) P[i] = __builtin_bit_cast(bf16x8, make_uint4(Pw[i][0], Pw[i][1], Pw[i][2], Pw[i][3]));
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
      const bf16x8 a = vfrag(Vt, db);
#pragma unroll
      for (int i = 0; i < NQB; ++i) O[db][i] = mfma_bf16(a, P[i], O[db][i]);
    }
#pragma unroll
    for (int i = 0; i < NQB; ++i) L[i] = mfma_bf16(ones, P[i], L[i]);
  }
#pragma unroll
  for (int i = 0; i < NQB; ++i) {
    const float inv = 1.0f / L[i][0];
    const int row = q0 + 16 * i + col;
    uint2 pk[4];
#pragma unroll
    for (int db = 0; db < 4; ++db)
      pk[db] = pack4_bf16_bits(O[db][i][0] * inv, O[db][i][1] * inv, O[db][i][2] * inv, O[db][i][3] * inv);
    store_tile_rows(ob + (size_t)(row < Sq ? row : 0) * HD, row < Sq, grp, pk);
  }
}

// grid: nqb * nbh blocks of 512 threads, block -> (b, h, query block) with the
// XCD-aware renumbering of attn_bf16_pipe
template <int NA, int NB>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_bf16_duo(const unsigned short* __restrict__ q, const unsigned short* __restrict__ k,
                   const unsigned short* __restrict__ v, unsigned short* __restrict__ o, int Sq, int Sk, float c,
                   int nbh) {
  __shared__ __align__(16) DuoLds sm;
  const int tid = threadIdx.x, w = tid >> 6;
  const int nqb = gridDim.x / nbh;
  const int nwg = gridDim.x, nwg8 = nwg & ~7;
  int item = blockIdx.x;
  if (item < nwg8) item = (item & 7) * (nwg8 >> 3) + (item >> 3);
  const size_t bh = item / nqb;
  const int base = (item % nqb) * (64 * (NA + NB));
  const unsigned short* qb = q + bh * (size_t)Sq * HD;
  const unsigned short* kb = k + bh * (size_t)Sk * HD;
  const unsigned short* vb = v + bh * (size_t)Sk * HD;
  unsigned short* ob = o + bh * (size_t)Sq * HD;
  if (w < 4)
    duo_wave<NA, false>(sm, qb, Sq, base + w * 16 * NA, kb, vb, Sk, c, ob, tid);
  else
    duo_wave<NB, false>(sm, qb, Sq, base + 64 * NA + (w - 4) * 16 * NB, kb, vb, Sk, c, ob, tid);
}

// 4-wave blocks, two per CU, for grids that fit one round: the launcher splits every head
// into items of s0 or s1 query units (a unit = one 16-query block per wave = 64 queries),
// round 0 (blocks [0, C)) takes the s0-items and round 1 the s1-items, so that block i and
// block i + C, which the dispatcher places on one CU, carry s0 + s1 units per SIMD.
// Heads [0, nX) split into aX s0-items and bX s1-items, the others into aY and bY.
struct QuadPlan {
  int c8;             // CUs / 8
  int s0, s1;         // units per item of round 0 / 1
  int nX, aX, bX, aY, bY;
  int cnt0, cnt1;     // items in round 0 / 1
};

__device__ __forceinline__ int quad_items(const QuadPlan& p, int r, int h) {
  return r == 0 ? (h < p.nX ? p.aX : p.aY) : (h < p.nX ? p.bX : p.bY);
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_bf16_quad(const unsigned short* __restrict__ q, const unsigned short* __restrict__ k,
                    const unsigned short* __restrict__ v, unsigned short* __restrict__ o, int Sq, int Sk, float c,
                    QuadPlan p) {
  __shared__ __align__(16) DuoLds sm;
  const int tid = threadIdx.x, w = tid >> 6;
  const int C = 8 * p.c8, r = blockIdx.x >= C, pi = blockIdx.x - r * C;
  // XCD-aware: block pi runs on XCD pi % 8, which takes items [c8 * (pi % 8), c8 * (pi % 8 + 1))
  const int l = (pi & 7) * p.c8 + (pi >> 3);
  if (l >= (r ? p.cnt1 : p.cnt0)) return;
  const int ax = quad_items(p, r, 0), ay = quad_items(p, r, p.nX);
  int h, j;
  if (l < p.nX * ax) {
    h = l / ax;
    j = l - h * ax;
  } else {
    const int l2 = l - p.nX * ax;
    h = p.nX + l2 / ay;
    j = l2 - (h - p.nX) * ay;
  }
  const int s = r ? p.s1 : p.s0;
  const int q0 = 64 * ((r ? quad_items(p, 0, h) * p.s0 : 0) + j * s);
  const size_t bh = h;
  const unsigned short* qb = q + bh * (size_t)Sq * HD;
  const unsigned short* kb = k + bh * (size_t)Sk * HD;
  const unsigned short* vb = v + bh * (size_t)Sk * HD;
  unsigned short* ob = o + bh * (size_t)Sq * HD;
  if (s == 3)
    duo_wave<3, true>(sm, qb, Sq, q0 + w * 48, kb, vb, Sk, c, ob, tid);
  else if (s == 2)
    duo_wave<2, true>(sm, qb, Sq, q0 + w * 32, kb, vb, Sk, c, ob, tid);
  else
    duo_wave<1, true>(sm, qb, Sq, q0 + w * 16, kb, vb, Sk, c, ob, tid);
}

// ---------------------------------------------------------------- bf16 cross (keys resident in LDS)
// Every key and value of a (b, h) is loaded into LDS once per workgroup and re-read by all
// its query blocks ("SDXL as a requirements inventory" s5.7: hold the re-read operand on
// chip, stream Q and O).  A workgroup serves a chunk of `qpc` queries of one (b, h): its
// waves take the chunk's 16-query blocks in turn, each requesting its next block's query
// rows while the current one computes.  Workgroups are numbered XCD-major so that the
// workgroups of one (b, h) share one XCD's L2.
//   ONLINE = false (NK <= 128): all scores of a query block in registers, one exact softmax.
//   ONLINE = true  (NK <= 512, the LDS budget): 64-key chunks out of LDS with a running
//   maximum and sum (the online softmax), O rescaled when the maximum rises.

// Workgroups are dispatched round-robin over the 8 XCDs: block b runs on XCD b % 8.  Map the
// first 8 * floor(n / 8) blocks so that XCD x takes a contiguous run of items.
__device__ __forceinline__ int xcd_major(int blk, int n) {
  const int n8 = n & ~7;
  return blk < n8 ? (blk & 7) * (n8 >> 3) + (blk >> 3) : blk;
}

template <int NK, int NW, bool ONLINE>
__global__ __launch_bounds__(64 * NW) void xattn_bf16(const unsigned short* __restrict__ q,
                                                      const unsigned short* __restrict__ k,
                                                      const unsigned short* __restrict__ v,
                                                      unsigned short* __restrict__ o, int Sq, int Sk, float c,
                                                      int nchunk, int qpc) {
  static_assert(NK % (ONLINE ? 64 : 32) == 0, "keys are consumed in 32-key (64-key online) steps");
  constexpr int NKB = NK / 16;
  __shared__ __align__(16) unsigned short Ks[NK * KP];
  __shared__ __align__(16) unsigned short Vs[NK * VP];
  constexpr int NT = 64 * NW;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int item = xcd_major(blockIdx.x, gridDim.x);
  const size_t bh = item / nchunk;
  const int qbase = (item % nchunk) * qpc;                  // qpc: a multiple of 16
  const int qend = min(Sq, qbase + qpc);
  const unsigned short* qb = q + bh * (size_t)Sq * HD;
  unsigned short* ob = o + bh * (size_t)Sq * HD;

  // this wave's query rows of its i-th block: qbase + 16 (i NW + w) + col; rows past Sq read as zero
  auto qload = [&](int i, bf16x8 (&Qf)[2]) {
    const int row = qbase + 16 * (i * NW + w) + col;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      uint4 u = make_uint4(0, 0, 0, 0);
      if (row < Sq) u = ld16(qb + (size_t)row * HD + 32 * t + 8 * grp);
      Qf[t] = __builtin_bit_cast(bf16x8, u);
    }
  };
  bf16x8 Qc[2], Qn[2];
  qload(0, Qc);
  bf16x8 ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = (__bf16)1.0f;
  {
    // every key and value of this (b, h); rows past Sk read as zero through the buffer
    // resources (their scores are masked)
    const rsrc_t krs = make_rsrc(k + bh * (size_t)Sk * HD, Sk * HD * 2);
    const rsrc_t vrs = make_rsrc(v + bh * (size_t)Sk * HD, Sk * HD * 2);
    constexpr int NIT = (NK * 8 + NT - 1) / NT;
    uint4 kk[NIT], vv[NIT];
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int idx = tid + it * NT;
      kk[it] = buf_ld16(krs, idx * 16);
      vv[it] = buf_ld16(vrs, idx * 16);
    }
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int idx = tid + it * NT, r = idx >> 3, cc = idx & 7;
      if (NIT * NT == NK * 8 || idx < NK * 8) {
        st16(&Ks[r * KP + cc * 8], kk[it]);
        st16(&Vs[r * VP + cc * 8], vv[it]);
      }
    }
  }
  __syncthreads();

  // ONLINE = false: the launcher gives every wave one block (qpc = 16 NW), so there is no loop
  for (int i = 0; ONLINE || i == 0; ++i) {
    const int q0 = qbase + 16 * (i * NW + w);
    if (q0 >= qend) break;  // wave-uniform; later blocks lie further on
    if (ONLINE && q0 + 16 * NW < qend) qload(i + 1, Qn);
    f32x4 O[4];
#pragma unroll
    for (int db = 0; db < 4; ++db) O[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    float l;
    if constexpr (!ONLINE) {
      f32x4 S[NKB];
#pragma unroll
      for (int kb_ = 0; kb_ < NKB; ++kb_) {
        const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(&Ks[(16 * kb_ + col) * KP + 8 * grp]);
        const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(&Ks[(16 * kb_ + col) * KP + 32 + 8 * grp]);
        S[kb_] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, Qc[0], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
        S[kb_] = mfma_bf16(a1, Qc[1], S[kb_]);
      }
      // padded keys are set to -inf before the maximum is taken; only a 16-key block that reaches
      // past Sk holds any (a wave-uniform test per block)
#pragma unroll
      for (int kb_ = 0; kb_ < NKB; ++kb_)
        if (16 * kb_ + 16 > Sk) {
#pragma unroll
          for (int e = 0; e < 4; ++e) S[kb_][e] = 16 * kb_ + 4 * grp + e < Sk ? S[kb_][e] : -INFINITY;
        }
      float mx = S[0][0];
#pragma unroll
      for (int kb_ = 0; kb_ < NKB; ++kb_)
#pragma unroll
        for (int e = 0; e < 4; ++e) mx = fmaxf(mx, S[kb_][e]);
      const float mc = group4_max(mx) * c;
#pragma unroll
      for (int kb_ = 0; kb_ < NKB; ++kb_)
#pragma unroll
        for (int e = 0; e < 4; ++e) S[kb_][e] = fast_exp2(__builtin_fmaf(S[kb_][e], c, -mc));
      // the row sum from an all-ones MFMA over the same bf16 weights as P.V
      f32x4 L = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < NKB / 2; ++ks) {
        const bf16x8 P = pack_bf16(S[2 * ks], S[2 * ks + 1]);
        const int vrow = 32 * ks + 4 * grp + (col >> 2);
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const int vcol = 16 * db + 4 * (col & 3);
          const bf16x8 a =
              cat_bf16(lds_read_tr16(&Vs[vrow * VP + vcol]), lds_read_tr16(&Vs[(vrow + 16) * VP + vcol]));
          O[db] = mfma_bf16(a, P, O[db]);
        }
        L = mfma_bf16(ones, P, L);
      }
      l = L[0];
    } else {
      float m = -INFINITY, lp = 0.0f;  // running maximum; this lane's share of the running sum
      const int nch = (Sk + 63) >> 6;
      for (int ch = 0; ch < nch; ++ch) {
        f32x4 S[4];
#pragma unroll
        for (int kb_ = 0; kb_ < 4; ++kb_) {
          const int r = 64 * ch + 16 * kb_ + col;
          const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(&Ks[r * KP + 8 * grp]);
          const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(&Ks[r * KP + 32 + 8 * grp]);
          S[kb_] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, Qc[0], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
          S[kb_] = mfma_bf16(a1, Qc[1], S[kb_]);
        }
        if (64 * ch + 64 > Sk) {
#pragma unroll
          for (int kb_ = 0; kb_ < 4; ++kb_)
#pragma unroll
            for (int e = 0; e < 4; ++e) S[kb_][e] = 64 * ch + 16 * kb_ + 4 * grp + e < Sk ? S[kb_][e] : -INFINITY;
        }
        float mx = S[0][0];
#pragma unroll
        for (int kb_ = 0; kb_ < 4; ++kb_)
#pragma unroll
          for (int e = 0; e < 4; ++e) mx = fmaxf(mx, S[kb_][e]);
        const float mnew = fmaxf(m, group4_max(mx));  // finite: chunk 0 holds key 0
        const float alpha = fast_exp2((m - mnew) * c);  // 0 on the first chunk
        const float mc = mnew * c;
        float ls = 0.0f;
#pragma unroll
        for (int kb_ = 0; kb_ < 4; ++kb_)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float p = fast_exp2(__builtin_fmaf(S[kb_][e], c, -mc));
            S[kb_][e] = p;
            ls += p;
          }
        lp = __builtin_fmaf(lp, alpha, ls);
        m = mnew;
#pragma unroll
        for (int db = 0; db < 4; ++db) O[db] *= alpha;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const bf16x8 P = pack_bf16(S[2 * ks], S[2 * ks + 1]);
          const int vrow = 64 * ch + 32 * ks + 4 * grp + (col >> 2);
#pragma unroll
          for (int db = 0; db < 4; ++db) {
            const int vcol = 16 * db + 4 * (col & 3);
            const bf16x8 a =
                cat_bf16(lds_read_tr16(&Vs[vrow * VP + vcol]), lds_read_tr16(&Vs[(vrow + 16) * VP + vcol]));
            O[db] = mfma_bf16(a, P, O[db]);
          }
        }
      }
      l = group4_sum(lp);
    }
    const float inv = 1.0f / l;
    const int row = q0 + col;
    uint2 pk[4];
#pragma unroll
    for (int db = 0; db < 4; ++db) pk[db] = pack4_bf16_bits(O[db][0] * inv, O[db][1] * inv, O[db][2] * inv, O[db][3] * inv);
    store_tile_rows(ob + (size_t)(row < Sq ? row : 0) * HD, row < Sq, grp, pk);
    if constexpr (ONLINE) {
      Qc[0] = Qn[0];
      Qc[1] = Qn[1];
    }
  }
}

// ---------------------------------------------------------------- launchers
hipError_t launch_attn_f32(const float* q, const float* k, const float* v, float* o, int B, int H, int Sq, int Sk,
                           float scale, hipStream_t s) {
  const int nqb = (Sq + F32_BQ - 1) / F32_BQ;
  hipLaunchKernelGGL(attn_f32_kernel, dim3(nqb * B * H), dim3(F32_BQ), 0, s, q, k, v, o, Sq, Sk, scale, nqb);
  return hipGetLastError();
}

namespace {
// compute units of the current device, cached per device (256 on MI355X).  Concurrent first
// calls may both query the attribute; they store the same value, and the accesses are atomic.
int cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

long long cdiv(long long a, long long b) { return (a + b - 1) / b; }

// per-SIMD query blocks x rounds of the best attn_bf16_duo layout, times the CU count
long long duo_cost(long long bh, int Sq, int cus) {
  const int na[3] = {3, 3, 2}, nb[3] = {3, 2, 2};
  long long best = -1;
  for (int i = 0; i < 3; ++i) {
    const long long cost = cdiv(bh * cdiv(Sq, 64 * (na[i] + nb[i])), cus) * (na[i] + nb[i]) * cus;
    if (best < 0 || cost < best) best = cost;
  }
  return best;
}

template <int NA, int NB>
hipError_t duo_launch(const unsigned short* q, const unsigned short* k, const unsigned short* v, unsigned short* o,
                      int B, int H, int Sq, int Sk, float c, hipStream_t s) {
  const int nqb = (int)cdiv(Sq, 64 * (NA + NB));
  hipLaunchKernelGGL((attn_bf16_duo<NA, NB>), dim3(nqb * B * H), dim3(512), 0, s, q, k, v, o, Sq, Sk, c, B * H);
  return hipGetLastError();
}
}  // namespace

// One-round plan for attn_bf16_quad: with U units per head and W = U * BH in all, each CU
// gets L = ceil(W / C) units per SIMD as an s0-item plus an s1-item.  Heads split into
// (aX, bX) or (aY, bY) items with s0 a + s1 b >= U; the counts must fit C per round.
// Least padding first, then the closest pair of splits: with every head split alike, the
// round-0 and round-1 items that an XCD takes come from the same heads (shared K / V in L2).
static bool quad_plan_search(long long bh, int Sq, int cus, QuadPlan& p) {
  if (cus % 8 != 0 || bh > 4 * (long long)cus) return false;
  const int U = (int)cdiv(Sq, 64);
  const long long L = cdiv(U * bh, cus);
  if (L < 4 || L > 6) return false;
  const int s0 = L == 4 ? 2 : 3, s1 = (int)L - s0;
  long long best = -1;
  const int amax = (int)cdiv(U, s0);
  for (int aX = 0; aX <= amax; ++aX)
    for (int aY = aX; aY <= amax; ++aY) {
      const int bX = (int)std::max(0LL, cdiv(U - s0 * aX, s1)), bY = (int)std::max(0LL, cdiv(U - s0 * aY, s1));
      for (long long nX = 0; nX <= bh; ++nX) {
        const long long A = nX * aX + (bh - nX) * aY, Bn = nX * bX + (bh - nX) * bY;
        if (A > cus || Bn > cus) continue;
        const long long waste = nX * (s0 * aX + s1 * bX) + (bh - nX) * (s0 * aY + s1 * bY) - U * bh;
        const long long score = waste * (amax + 1) + (aY - aX);
        if (best < 0 || score < best) {
          best = score;
          p = QuadPlan{cus / 8, s0, s1, (int)nX, aX, bX, aY, bY, (int)A, (int)Bn};
        }
      }
    }
  return best >= 0;
}

// the search is small (L <= 6 bounds U * BH) but runs per launch: remember the last shape
static bool quad_plan(long long bh, int Sq, int cus, QuadPlan& p) {
  thread_local long long key_bh = -1;
  thread_local int key_sq = -1, key_cus = -1;
  thread_local bool ok = false;
  thread_local QuadPlan plan{};
  if (bh != key_bh || Sq != key_sq || cus != key_cus) {
    ok = quad_plan_search(bh, Sq, cus, plan);
    key_bh = bh;
    key_sq = Sq;
    key_cus = cus;
  }
  p = plan;
  return ok;
}

// Which bf16 head-dim-64 kernel (and layout) a call of this shape runs on `cus` CUs.
enum DenseKind { DK_QUAD, DK_DUO33, DK_DUO32, DK_DUO22, DK_PIPE };
static DenseKind choose_dense(long long bh, int Sq, int cus, QuadPlan& plan) {
  if (quad_plan(bh, Sq, cus, plan) && (long long)(plan.s0 + plan.s1) * cus < duo_cost(bh, Sq, cus)) return DK_QUAD;
  if (bh * cdiv(Sq, 256) >= cus) {
    // one 8-wave block per CU: pick the query blocks per SIMD (NA + NB) that minimise
    // rounds x per-SIMD work, e.g. 3+3 (one round of 220 blocks) for B=2, H=10, S=4096
    const int na[3] = {3, 3, 2}, nb[3] = {3, 2, 2};
    int best = 0;
    long long best_cost = -1;
    for (int i = 0; i < 3; ++i) {
      const long long cost = cdiv(bh * cdiv(Sq, 64 * (na[i] + nb[i])), cus) * (na[i] + nb[i]);
      if (best_cost < 0 || cost < best_cost) { best = i; best_cost = cost; }
    }
    return best == 0 ? DK_DUO33 : best == 1 ? DK_DUO32 : DK_DUO22;
  }
  return DK_PIPE;  // small grids: 16 queries per wave, 4 waves per block, 4 waves per SIMD
}

hipError_t launch_attn_bf16(const unsigned short* q, const unsigned short* k, const unsigned short* v,
                            unsigned short* o, int B, int H, int Sq, int Sk, float scale, hipStream_t s) {
  const float c = scale * LOG2E;
  QuadPlan plan;
  switch (choose_dense((long long)B * H, Sq, cu_count(), plan)) {
    case DK_QUAD:
      hipLaunchKernelGGL(attn_bf16_quad, dim3(16 * plan.c8), dim3(256), 0, s, q, k, v, o, Sq, Sk, c, plan);
      return hipGetLastError();
    case DK_DUO33: return duo_launch<3, 3>(q, k, v, o, B, H, Sq, Sk, c, s);
    case DK_DUO32: return duo_launch<3, 2>(q, k, v, o, B, H, Sq, Sk, c, s);
    case DK_DUO22: return duo_launch<2, 2>(q, k, v, o, B, H, Sq, Sk, c, s);
    case DK_PIPE: break;
  }
  constexpr int NQB = 1, NW = 4;
  const int nqb = (Sq + 16 * NQB * NW - 1) / (16 * NQB * NW);
  dim3 grid(nqb * B * H);  // one dimension: the kernel maps block -> (b, h, query block)
  hipLaunchKernelGGL((attn_bf16_pipe<NQB, NW, 0, 4>), grid, dim3(64 * NW), 0, s, q, k, v, o, Sq, Sk, c, B * H);
  return hipGetLastError();
}

const char* attn_bf16_kernel_name(int B, int H, int Sq) {
  QuadPlan plan;
  switch (choose_dense((long long)B * H, Sq, cu_count(), plan)) {
    case DK_QUAD:
      return plan.s0 == 3 ? (plan.s1 == 3 ? "attn_bf16_quad 3+3" : "attn_bf16_quad 3+2")
                          : "attn_bf16_quad 2+2";
    case DK_DUO33: return "attn_bf16_duo 3+3";
    case DK_DUO32: return "attn_bf16_duo 3+2";
    case DK_DUO22: return "attn_bf16_duo 2+2";
    case DK_PIPE: break;
  }
  return "attn_bf16_pipe";
}

// Query chunks per (b, h).  Up to 128 keys a workgroup is small (<= 39 KB of LDS, four waves)
// and several share a CU, so every wave takes one 16-query block: the most workgroups, whose
// latencies overlap.  Larger key sets fill most of a CU's LDS (one workgroup per CU): then the
// chunks are sized so that all workgroups fit one round on the chip.
static void xattn_chunks(long long bh, int Sq, int nw, bool big, int cus, int& nchunk, int& qpc) {
  const long long nblk = cdiv(Sq, 16);
  long long n = big ? std::max(1LL, cus / bh) : cdiv(nblk, nw);  // not big: one block per wave
  n = std::min(n, nblk);
  qpc = (int)(16 * cdiv(nblk, n));
  nchunk = (int)cdiv(Sq, qpc);
}

template <int NK, int NW, bool ONLINE>
static hipError_t xlaunch(const unsigned short* q, const unsigned short* k, const unsigned short* v,
                          unsigned short* o, int B, int H, int Sq, int Sk, float c, hipStream_t s) {
  const long long bh = (long long)B * H;
  int nchunk = 1, qpc = 16;
  xattn_chunks(bh, Sq, NW, ONLINE && NK > 256, cu_count(), nchunk, qpc);
  hipLaunchKernelGGL((xattn_bf16<NK, NW, ONLINE>), dim3((unsigned)(bh * nchunk)), dim3(64 * NW), 0, s, q, k, v, o,
                     Sq, Sk, c, nchunk, qpc);
  return hipGetLastError();
}

hipError_t launch_xattn_bf16(const unsigned short* q, const unsigned short* k, const unsigned short* v,
                             unsigned short* o, int B, int H, int Sq, int Sk, float scale, hipStream_t s) {
  const float c = scale * LOG2E;
  // up to 128 keys: every score of a query block in registers, one exact pass; longer key sets
  // (up to the LDS budget, KA_XATTN_MAX_SK) in 64-key chunks out of LDS with an online softmax.
  // Past 256 keys one workgroup fills most of a CU's LDS: sixteen waves, four per SIMD.
  if (Sk <= 32) return xlaunch<32, 4, false>(q, k, v, o, B, H, Sq, Sk, c, s);
  if (Sk <= 64) return xlaunch<64, 4, false>(q, k, v, o, B, H, Sq, Sk, c, s);
  if (Sk <= 96) return xlaunch<96, 4, false>(q, k, v, o, B, H, Sq, Sk, c, s);
  if (Sk <= 128) return xlaunch<128, 4, false>(q, k, v, o, B, H, Sq, Sk, c, s);
  if (Sk <= 192) return xlaunch<192, 4, true>(q, k, v, o, B, H, Sq, Sk, c, s);
  if (Sk <= 256) return xlaunch<256, 4, true>(q, k, v, o, B, H, Sq, Sk, c, s);
  if (Sk <= 320) return xlaunch<320, 16, true>(q, k, v, o, B, H, Sq, Sk, c, s);
  if (Sk <= 384) return xlaunch<384, 16, true>(q, k, v, o, B, H, Sq, Sk, c, s);
  if (Sk <= 448) return xlaunch<448, 16, true>(q, k, v, o, B, H, Sq, Sk, c, s);
  return xlaunch<512, 16, true>(q, k, v, o, B, H, Sq, Sk, c, s);
}

}  // namespace ka
