// attn512.hip -- dense attention at head dim 512 for gfx950: the SDXL VAE's mid-block
// AttnBlock, one head of 512 channels over the 128 x 128 latent grid (16384 tokens)
// ("SDXL as a requirements inventory", s1.5 and s5.10).
//
// The same flash loop as the head-dim-64 kernels, S^T = K Q^T and O^T = V^T P^T with the
// softmax statistics of a query in one lane group, with everything eight times wider in D:
//   - a wave owns 16 queries: its Q^T operand is 16 k-steps of 32 dims (64 VGPRs) and its
//     O^T accumulator 32 tiles of 16 dims (128 VGPRs; this file is built with the matrix
//     instructions' VGPR form, so the rare rescale needs no AGPR copies);
//   - the running maximum is raised lazily (LAZY_LOG2), so O is rescaled only on a raise;
//   - the loop is bound by the LDS reads of the K and V fragments: every wave reads a whole
//     tile of each for its 16 queries (64 bytes of LDS per key and dim pair of K and V).
#include "ka_common.hpp"
#include "ka_kernels.hpp"

namespace ka {

constexpr int D5 = 512;           // head dim
constexpr int KP5 = D5 + 8;       // LDS pitch of K (elements): rows 4 banks apart for the b128 fragment reads
constexpr int VP5 = D5 + 16;      // LDS pitch of V (elements), as VP for the transposed reads

// Two waves per SIMD by splitting the keys: a block of eight waves serves 64 queries, waves w and
// w + 4 the same 16 (w % 4), wave w taking the even and wave w + 4 the odd 16-key tiles of
// every 32 keys.  Each half has its own double-buffered K and V tiles in LDS (134 KB in all: one
// block per CU, 256 blocks for the 16384-token head), so the second wave of a SIMD covers the
// first one's LDS and MFMA latencies.  Per 16-key tile a wave issues 16 MFMAs 16x16x32 for S^T and 32 MFMAs 16x16x16
// for O^T (the weights of 16 keys are one B operand).  At the end the odd-tile waves leave
// (m, l, O) in LDS and the even-tile waves merge them with the online-softmax rescale.
constexpr int BP5 = 16;  // keys per tile and half
#ifndef A512_PF
#define A512_PF 2
#endif
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
      // S^T of the 16 keys: two accumulation chains (even and odd k-steps), the K fragments read
      // A512_PF k-steps ahead of their MFMA
      f32x4 S2[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
      bf16x8 kf[A512_PF];
      auto kread = [&](int ks) { return *reinterpret_cast<const bf16x8*>(&Kt[col * KP5 + 32 * ks + 8 * grp]); };
#pragma unroll
      for (int i = 0; i < A512_PF; ++i) kf[i] = kread(i);
#pragma unroll
      for (int ks = 0; ks < D5 / 32; ++ks) {
        const bf16x8 a = kf[ks % A512_PF];
        if (ks + A512_PF < D5 / 32) kf[ks % A512_PF] = kread(ks + A512_PF);
        S2[ks & 1] = mfma_bf16(a, Qf[ks], S2[ks & 1]);
        __builtin_amdgcn_sched_barrier(0);
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
  // O as [4 waves][32 dim blocks][64 lanes] f32x4 (a wave's accesses to one block are one
  // contiguous 1 KB, free of bank conflicts), then m and l as [4][64][2]
  f32x4* XO = reinterpret_cast<f32x4*>(&sm);
  static_assert(sizeof(LdsPair512) >= 4 * 64 * (D5 / 4 + 2) * 4, "the merge area fits the tiles");
  auto xo = [&](int db) -> f32x4& { return XO[(wq * (D5 / 16) + db) * 64 + lane]; };
  float* xm = reinterpret_cast<float*>(XO + 4 * (D5 / 16) * 64) + 2 * (wq * 64 + lane);
  if (half) {
    xm[0] = m;
    xm[1] = L[0];
#pragma unroll
    for (int db = 0; db < D5 / 16; ++db) xo(db) = O[db];
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
      const f32x4 o1 = xo(db);
      f32x4 r;
#pragma unroll
      for (int e = 0; e < 4; ++e) r[e] = (O[db][e] * a0 + o1[e] * a1) * inv;
      st8(ob + (size_t)row * D5 + 16 * db + 4 * grp, pack4_bf16_bits(r[0], r[1], r[2], r[3]));
    }
  }
}

hipError_t launch_attn512_bf16(const unsigned short* q, const unsigned short* k, const unsigned short* v,
                               unsigned short* o, int B, int H, int Sq, int Sk, float scale, hipStream_t s) {
  const int nqb = (Sq + 63) / 64;
  hipLaunchKernelGGL(attn512_pair, dim3(nqb * B * H), dim3(512), 0, s, q, k, v, o, Sq, Sk, scale * LOG2E, nqb);
  return hipGetLastError();
}

}  // namespace ka
