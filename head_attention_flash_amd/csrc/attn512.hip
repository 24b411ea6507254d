// attn512.hip -- dense attention at head dim 512 for gfx950: the SDXL VAE's mid-block
// AttnBlock, one head of 512 channels over the 128 x 128 latent grid (16384 tokens)
// ("SDXL as a requirements inventory", s1.5 and s5.10).
//
// The same flash loop as the head-dim-64 kernels, S^T = K Q^T and O^T = V^T P^T on
// v_mfma_f32_16x16x32_bf16 with the softmax statistics of a query in one lane group,
// with everything eight times wider in D:
//   - a wave owns 16 queries: its Q^T operand is 16 k-steps of 32 dims (64 VGPRs) and
//     its O^T accumulator 32 tiles of 16 dims (128 VGPRs: this file is built with the
//     matrix instructions' VGPR form, since AGPR accumulators were copied to VGPRs and
//     back every tile for the rescale);
//   - a block of four waves (64 queries) shares 32-key K and V tiles of 32 KB each in
//     LDS, double-buffered (134 KB: one block per CU).  Tiles go from HBM straight into
//     LDS (global_load_lds_dwordx4: one wave instruction moves one 1 KB row, lane i's 16
//     bytes landing at row base + 16 i), issued one tile ahead, so no registers hold
//     staged data and O and Q^T fit the VGPRs together;
//   - per 32-key tile a wave issues 32 MFMAs for S^T and 32 (plus one row-sum MFMA) for
//     O^T; the softmax is 8 exponentials per lane, an eighth of the matrix work's issue
//     time at D = 64's ratio, so the loop is bound by the matrix core and by the LDS
//     reads of the K and V fragments (64 KB per wave and tile).
//   - the running maximum is raised lazily (LAZY_LOG2), so O is rescaled only on a raise.
#include "ka_common.hpp"
#include "ka_kernels.hpp"

namespace ka {

constexpr int D5 = 512;           // head dim
constexpr int BN5 = 32;           // keys per tile
constexpr int KP5 = D5 + 8;       // LDS pitch of K (elements): rows 4 banks apart for the b128 fragment reads
constexpr int VP5 = D5 + 16;      // LDS pitch of V (elements), as VP for the transposed reads

// LDS pointer for the direct global-to-LDS loads
typedef __attribute__((address_space(3))) void lds_void;

struct Lds512 {
  unsigned short K[2][BN5 * KP5];
  unsigned short V[2][BN5 * VP5];
};

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn512_bf16(const unsigned short* __restrict__ q, const unsigned short* __restrict__ k,
                  const unsigned short* __restrict__ v, unsigned short* __restrict__ o, int Sq, int Sk, float c,
                  int nqb) {
  __shared__ __align__(16) Lds512 sm;
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const size_t bh = blockIdx.x / nqb;  // one-dimensional grid: (b, h) major, 64-query block minor
  const unsigned short* qb = q + bh * (size_t)Sq * D5;
  unsigned short* ob = o + bh * (size_t)Sq * D5;
  const int q0 = (blockIdx.x % nqb) * 64 + 16 * w;

  // Q^T (B operand): k-step ks covers dims 32 ks + 8 grp .. + 8 of query q0 + col
  bf16x8 Qf[D5 / 32];
  {
    const int row = q0 + col;
#pragma unroll
    for (int ks = 0; ks < D5 / 32; ++ks) {
      uint4 u = make_uint4(0, 0, 0, 0);
      if (row < Sq) u = ld16(qb + (size_t)row * D5 + 32 * ks + 8 * grp);
      Qf[ks] = __builtin_bit_cast(bf16x8, u);
    }
  }
  f32x4 O[D5 / 16];
#pragma unroll
  for (int db = 0; db < D5 / 16; ++db) O[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 L = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY;
  bf16x8 ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = (__bf16)1.0f;

  // tile t into LDS buffer `buf`: wave w moves rows w, w + 4, ... of K and of V, one 1 KB row
  // per instruction; rows past Sk repeat row Sk - 1 (their scores are masked, their weights 0)
  const unsigned short* kb = k + bh * (size_t)Sk * D5;
  const unsigned short* vb = v + bh * (size_t)Sk * D5;
  auto tile_load = [&](int t, int buf) {
#pragma unroll
    for (int i = 0; i < BN5 / 4; ++i) {
      const int row = w + 4 * i;
      const size_t j = (size_t)min(t * BN5 + row, Sk - 1);
      __builtin_amdgcn_global_load_lds(kb + j * D5 + 8 * lane, (lds_void*)&sm.K[buf][row * KP5], 16, 0, 0);
      __builtin_amdgcn_global_load_lds(vb + j * D5 + 8 * lane, (lds_void*)&sm.V[buf][row * VP5], 16, 0, 0);
    }
  };

  const int T = (Sk + BN5 - 1) / BN5;
  tile_load(0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int t = 0; t < T; ++t) {
    const int cur = t & 1;
    if (t + 1 < T) tile_load(t + 1, cur ^ 1);  // that buffer was last read in step t - 1
    const unsigned short* Kt = sm.K[cur];
    const unsigned short* Vt = sm.V[cur];
    // S^T for two 16-key blocks: four independent accumulation chains (even and odd k-steps)
    f32x4 S4[2][2] = {{f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}},
                      {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}}};
#pragma unroll
    for (int ks = 0; ks < D5 / 32; ++ks) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(&Kt[(16 * kb + col) * KP5 + 32 * ks + 8 * grp]);
        S4[kb][ks & 1] = mfma_bf16(a, Qf[ks], S4[kb][ks & 1]);
      }
    }
    f32x4 S[2] = {S4[0][0] + S4[0][1], S4[1][0] + S4[1][1]};
    if ((t + 1) * BN5 > Sk) {  // tail tile (uniform): keys past Sk take no weight
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 4; ++e) S[kb][e] = t * BN5 + 16 * kb + 4 * grp + e < Sk ? S[kb][e] : -INFINITY;
    }
    float mx = fmaxf(fmaxf(fmaxf(S[0][0], S[0][1]), fmaxf(S[0][2], S[0][3])),
                     fmaxf(fmaxf(S[1][0], S[1][1]), fmaxf(S[1][2], S[1][3])));
    mx = group4_max(mx);
    const bool raise = (mx - m) * c > LAZY_LOG2;  // true on the first tile (m = -inf)
    const float mnew = raise ? mx : m;
    const float alpha = fast_exp2((m - mnew) * c);  // 1 when not raised
    m = mnew;
    const float mc = mnew * c;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 4; ++e) S[kb][e] = fast_exp2(__builtin_fmaf(S[kb][e], c, -mc));
    if (__builtin_amdgcn_ballot_w64(raise)) {
#pragma unroll
      for (int db = 0; db < D5 / 16; ++db) O[db] *= alpha;
      L *= alpha;
    }
    // P^T (B operand): keys 4 grp + e of the first 16-key block, then of the second
    const bf16x8 P = pack_bf16(S[0], S[1]);
    // V^T (A operand): lane row = dim 16 db + (lane % 16), k = the keys in P^T's order
    const int vrow = 4 * grp + (col >> 2);
#pragma unroll
    for (int db = 0; db < D5 / 16; ++db) {
      const int vcol = 16 * db + 4 * (col & 3);
      const bf16x8 a = cat_bf16(lds_read_tr16(&Vt[vrow * VP5 + vcol]), lds_read_tr16(&Vt[(vrow + 16) * VP5 + vcol]));
      O[db] = mfma_bf16(a, P, O[db]);
    }
    L = mfma_bf16(ones, P, L);
    __builtin_amdgcn_s_waitcnt(0);  // the next tile has landed in LDS
    __syncthreads();
  }

  const int row = q0 + col;
  if (row < Sq) {
    const float inv = 1.0f / L[0];
#pragma unroll
    for (int db = 0; db < D5 / 16; ++db)
      st8(ob + (size_t)row * D5 + 16 * db + 4 * grp,
          pack4_bf16_bits(O[db][0] * inv, O[db][1] * inv, O[db][2] * inv, O[db][3] * inv));
  }
}

// Two waves per SIMD by splitting the keys: a block of eight waves serves 64 queries, waves w and
// w + 4 the same 16 (w % 4), wave w taking the even and wave w + 4 the odd 16-key tiles of
// every 32 keys.  Each half has its own double-buffered K and V tiles in LDS (134 KB in all, one
// block per CU as before), so the second wave of a SIMD covers the first one's LDS and MFMA
// latencies.  Per 16-key tile a wave issues 16 MFMAs 16x16x32 for S^T and 32 MFMAs 16x16x16
// for O^T (the weights of 16 keys are one B operand).  At the end the odd-tile waves leave
// (m, l, O) in LDS and the even-tile waves merge them with the online-softmax rescale.
constexpr int BP5 = 16;  // keys per tile and half
typedef __attribute__((ext_vector_type(4))) short s16x4;
struct LdsPair512 {
  unsigned short K[2][2][BP5 * KP5];  // [half][buffer]
  unsigned short V[2][2][BP5 * VP5];
};

__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn512_pair(const unsigned short* __restrict__ q, const unsigned short* __restrict__ k,
                  const unsigned short* __restrict__ v, unsigned short* __restrict__ o, int Sq, int Sk, float c,
                  int nqb) {
  __shared__ __align__(16) LdsPair512 sm;
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const int half = w >> 2, wq = w & 3;  // key-tile parity; query block of the wave
  const size_t bh = blockIdx.x / nqb;
  const unsigned short* qb = q + bh * (size_t)Sq * D5;
  unsigned short* ob = o + bh * (size_t)Sq * D5;
  const int q0 = (blockIdx.x % nqb) * 64 + 16 * wq;

  bf16x8 Qf[D5 / 32];
  {
    const int row = q0 + col;
#pragma unroll
    for (int ks = 0; ks < D5 / 32; ++ks) {
      uint4 u = make_uint4(0, 0, 0, 0);
      if (row < Sq) u = ld16(qb + (size_t)row * D5 + 32 * ks + 8 * grp);
      Qf[ks] = __builtin_bit_cast(bf16x8, u);
    }
  }
  f32x4 O[D5 / 16];
#pragma unroll
  for (int db = 0; db < D5 / 16; ++db) O[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 L = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY;
  s16x4 ones;
#pragma unroll
  for (int e = 0; e < 4; ++e) ones[e] = (short)0x3F80;  // bf16 1.0

  // tile tt (16 keys) of this half into buffer buf: the half's four waves move rows wq, wq + 4, ..
  // of K and V, one 1 KB row per instruction (lane l's 16 bytes at the row base + 16 l); rows
  // past Sk read as zero through the descriptors (their scores are masked).  Inline assembly with
  // the tile offset in the descriptor and the slot in M0: the compiler does not make the V reads
  // of the current tile wait for the next tile's loads.
  const int T16 = (Sk + BP5 - 1) / BP5;          // 16-key tiles
  const int NS = (T16 + 1) / 2;                  // steps: tiles 2s (half 0) and 2s + 1 (half 1)
  const u32x4_t krs = raw_rsrc(k + bh * (size_t)Sk * D5, Sk * D5 * 2);
  const u32x4_t vrs = raw_rsrc(v + bh * (size_t)Sk * D5, Sk * D5 * 2);
  const unsigned ldsK = lds_addr(&sm.K[half][0][0]), ldsV = lds_addr(&sm.V[half][0][0]);
  constexpr unsigned KT = BP5 * KP5 * 2, VT = BP5 * VP5 * 2;  // bytes of a tile buffer
  auto tile_load = [&](int tt, int buf) {
    const u32x4_t kr = rsrc_advance(krs, (unsigned)tt * (BP5 * D5 * 2));
    const u32x4_t vr = rsrc_advance(vrs, (unsigned)tt * (BP5 * D5 * 2));
#pragma unroll
    for (int i = 0; i < BP5 / 4; ++i) {
      const int row = wq + 4 * i;
      load16_to_lds(kr, row * (D5 * 2) + 16 * lane, ldsK + buf * KT + row * (KP5 * 2));
      load16_to_lds(vr, row * (D5 * 2) + 16 * lane, ldsV + buf * VT + row * (VP5 * 2));
    }
  };
  if (half < T16) tile_load(half, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int s = 0; s < NS; ++s) {
    const int cur = s & 1, tt = 2 * s + half;
    if (tt + 2 < T16) tile_load(tt + 2, cur ^ 1);  // that buffer was last read in step s - 1
    if (tt < T16) {  // wave-uniform: the odd half has no tile in the last step of an odd count
      const unsigned short* Kt = sm.K[half][cur];
      const unsigned short* Vt = sm.V[half][cur];
      // S^T of the 16 keys: two accumulation chains (even and odd k-steps)
      f32x4 S2[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int ks = 0; ks < D5 / 32; ++ks) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(&Kt[col * KP5 + 32 * ks + 8 * grp]);
        S2[ks & 1] = mfma_bf16(a, Qf[ks], S2[ks & 1]);
      }
      f32x4 S = S2[0] + S2[1];
      if ((tt + 1) * BP5 > Sk) {  // tail tile (uniform): keys past Sk take no weight
#pragma unroll
        for (int e = 0; e < 4; ++e) S[e] = tt * BP5 + 4 * grp + e < Sk ? S[e] : -INFINITY;
      }
      float mx = group4_max(fmaxf(fmaxf(S[0], S[1]), fmaxf(S[2], S[3])));
      const bool raise = (mx - m) * c > LAZY_LOG2;  // true on the first tile (m = -inf)
      const float mnew = raise ? mx : m;
      const float alpha = fast_exp2((m - mnew) * c);  // 1 when not raised
      m = mnew;
      const float mc = mnew * c;
#pragma unroll
      for (int e = 0; e < 4; ++e) S[e] = fast_exp2(__builtin_fmaf(S[e], c, -mc));
      if (__builtin_amdgcn_ballot_w64(raise)) {
#pragma unroll
        for (int db = 0; db < D5 / 16; ++db) O[db] *= alpha;
        L *= alpha;
      }
      // P^T (B operand, 16 keys): keys 4 grp + e of the tile; V^T (A operand): lane row = dim
      // 16 db + (lane % 16), k = the same keys
      const s16x4 P = __builtin_bit_cast(s16x4, pack4_bf16_bits(S[0], S[1], S[2], S[3]));
      const int vrow = 4 * grp + (col >> 2);
#pragma unroll
      for (int db = 0; db < D5 / 16; ++db) {
        const s16x4 a = __builtin_bit_cast(s16x4, lds_read_tr16(&Vt[vrow * VP5 + 16 * db + 4 * (col & 3)]));
        O[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, P, O[db], 0, 0, 0);
      }
      L = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ones, P, L, 0, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(0);  // the next tiles have landed in LDS
    __syncthreads();
  }

  // merge: the odd-tile waves leave m, l and O in LDS (over the tile buffers, no longer read after
  // the last barrier); the even-tile waves rescale both to the larger maximum and add
  // [4 waves][64 lanes][128] O (16-byte aligned rows), then [4][64][2] m and l
  float* X = reinterpret_cast<float*>(&sm);
  static_assert(sizeof(LdsPair512) >= 4 * 64 * (D5 / 4 + 2) * 4, "the merge area fits the tiles");
  const int xi = wq * 64 + lane;
  float* xo = X + (size_t)xi * (D5 / 4);
  float* xm = X + 4 * 64 * (D5 / 4) + 2 * xi;
  if (half) {
    xm[0] = m;
    xm[1] = L[0];
#pragma unroll
    for (int db = 0; db < D5 / 16; ++db) *reinterpret_cast<f32x4*>(&xo[4 * db]) = O[db];
  }
  __syncthreads();
  if (half) return;
  const float m1 = xm[0], l1 = xm[1];
  const float mt = fmaxf(m, m1);                       // m is finite: tile 0 is the even half's
  const float a0 = fast_exp2((m - mt) * c), a1 = fast_exp2((m1 - mt) * c);  // a1 = 0 if the odd half saw no key
  const float inv = 1.0f / (L[0] * a0 + l1 * a1);
  const int row = q0 + col;
  if (row < Sq) {
#pragma unroll
    for (int db = 0; db < D5 / 16; ++db) {
      const f32x4 o1 = *reinterpret_cast<const f32x4*>(&xo[4 * db]);
      f32x4 r;
#pragma unroll
      for (int e = 0; e < 4; ++e) r[e] = (O[db][e] * a0 + o1[e] * a1) * inv;
      st8(ob + (size_t)row * D5 + 16 * db + 4 * grp, pack4_bf16_bits(r[0], r[1], r[2], r[3]));
    }
  }
}

#ifndef A512_PAIR
#define A512_PAIR 1
#endif
hipError_t launch_attn512_bf16(const unsigned short* q, const unsigned short* k, const unsigned short* v,
                               unsigned short* o, int B, int H, int Sq, int Sk, float scale, hipStream_t s) {
  const int nqb = (Sq + 63) / 64;
  if (A512_PAIR)
    hipLaunchKernelGGL(attn512_pair, dim3(nqb * B * H), dim3(512), 0, s, q, k, v, o, Sq, Sk, scale * LOG2E, nqb);
  else
    hipLaunchKernelGGL(attn512_bf16, dim3(nqb * B * H), dim3(256), 0, s, q, k, v, o, Sq, Sk, scale * LOG2E, nqb);
  return hipGetLastError();
}

}  // namespace ka
