// attn512.hip -- dense attention at head dim 512 for gfx950: the SDXL VAE's mid-block
// AttnBlock, one head of 512 channels over the 128 x 128 latent grid (16384 tokens)
// ("SDXL as a requirements inventory", s1.5 and s5.10).
//
// The same flash loop as the head-dim-64 kernels, S^T = K Q^T and O^T = V^T P^T on
// v_mfma_f32_16x16x32_bf16 with the softmax statistics of a query in one lane group,
// with everything eight times wider in D:
//   - a wave owns 16 queries: its Q^T operand is 16 k-steps of 32 dims (64 VGPRs) and
//     its O^T accumulator 32 tiles of 16 dims (128 registers, which the compiler keeps
//     in AGPRs);
//   - a block of four waves (64 queries) shares 32-key K and V tiles of 32 KB each in
//     LDS, double-buffered (134 KB: one block per CU); each thread stages 8 + 8 chunks
//     of 16 bytes per tile through registers, loaded one tile ahead;
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
constexpr int CH5 = BN5 * D5 / 8 / 256;  // 16-byte chunks per thread and tensor per tile (8)

struct Lds512 {
  unsigned short K[2][BN5 * KP5];
  unsigned short V[2][BN5 * VP5];
};

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn512_bf16(const unsigned short* __restrict__ q, const unsigned short* __restrict__ k,
                  const unsigned short* __restrict__ v, unsigned short* __restrict__ o, int Sq, int Sk, float c) {
  __shared__ __align__(16) Lds512 sm;
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const size_t bh = blockIdx.y;
  const unsigned short* qb = q + bh * (size_t)Sq * D5;
  unsigned short* ob = o + bh * (size_t)Sq * D5;
  // keys and values past Sk read as zero through the buffer resources (their scores are masked)
  const rsrc_t krs = make_rsrc(k + bh * (size_t)Sk * D5, Sk * D5 * 2);
  const rsrc_t vrs = make_rsrc(v + bh * (size_t)Sk * D5, Sk * D5 * 2);
  const int q0 = blockIdx.x * 64 + 16 * w;

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

  // tile staging: chunk tid + 256 it is row (tid + 256 it) / 64, 16-byte column (tid & 63)
  uint4 sk[CH5], sv[CH5];
  auto gload = [&](int t) {
#pragma unroll
    for (int it = 0; it < CH5; ++it) {
      const int off = t * (BN5 * D5 * 2) + (tid + 256 * it) * 16;
      sk[it] = buf_ld16(krs, off);
      sv[it] = buf_ld16(vrs, off);
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int it = 0; it < CH5; ++it) {
      const int row = (tid >> 6) + 4 * it, c8 = (tid & 63) * 8;
      st16(&sm.K[buf][row * KP5 + c8], sk[it]);
      st16(&sm.V[buf][row * VP5 + c8], sv[it]);
    }
  };

  const int T = (Sk + BN5 - 1) / BN5;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int t = 0; t < T; ++t) {
    const int cur = t & 1;
    if (t + 1 < T) gload(t + 1);
    const unsigned short* Kt = sm.K[cur];
    const unsigned short* Vt = sm.V[cur];
    // S^T for two 16-key blocks, 16 k-steps each (two independent accumulation chains)
    f32x4 S[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int ks = 0; ks < D5 / 32; ++ks) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(&Kt[(16 * kb + col) * KP5 + 32 * ks + 8 * grp]);
        S[kb] = mfma_bf16(a, Qf[ks], S[kb]);
      }
    }
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
    if (t + 1 < T) lstore(cur ^ 1);  // that buffer was last read in step t - 1
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

hipError_t launch_attn512_bf16(const unsigned short* q, const unsigned short* k, const unsigned short* v,
                               unsigned short* o, int B, int H, int Sq, int Sk, float scale, hipStream_t s) {
  dim3 grid((Sq + 63) / 64, B * H);
  hipLaunchKernelGGL(attn512_bf16, grid, dim3(256), 0, s, q, k, v, o, Sq, Sk, scale * LOG2E);
  return hipGetLastError();
}

}  // namespace ka
