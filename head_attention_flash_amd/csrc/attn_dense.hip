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
//   attn_bf16_flash<..>    bf16 in/out; S^T = K Q^T and O^T = V^T P^T on
//                          v_mfma_f32_16x16x32_bf16, fp32 softmax; K/V tiles of 64
//                          keys double-buffered in LDS; the 1/sum is applied once
//                          per output row after P.V (the "divide after P.V" trim of
//                          "401 -> 163 ms: Stable Audio 3 medium on one TPU v6e
//                          chip", s4).
//   xattn_bf16<..>         cross-attention for short key sets: every key and value
//                          of a (b, h) is loaded into LDS once and re-read by every
//                          query tile ("SDXL as a requirements inventory" s5.7: hold
//                          the re-read operand, stream Q/O); one exact softmax pass.
#include "ka_common.hpp"
#include "ka_kernels.hpp"

namespace ka {

// ---------------------------------------------------------------- fp32
constexpr int F32_BQ = 128;  // queries per block (one per thread)
constexpr int F32_BK = 32;   // keys per LDS tile

__global__ __launch_bounds__(F32_BQ) void attn_f32_kernel(const float* __restrict__ q, const float* __restrict__ k,
                                                          const float* __restrict__ v, float* __restrict__ o, int Sq,
                                                          int Sk, float scale) {
  __shared__ __align__(16) float ks[F32_BK][HD];
  __shared__ __align__(16) float vs[F32_BK][HD];
  const int tid = threadIdx.x;
  const size_t bh = blockIdx.y;
  const int i = blockIdx.x * F32_BQ + tid;
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

// ---------------------------------------------------------------- bf16 flash
// LDS pitches (in 16-bit elements): K rows are read as 16-byte A-operand chunks,
// V rows through the transposed 8-byte read; both pitches keep a wave's reads on
// distinct banks.
constexpr int KP = HD + 8;
constexpr int VP = HD + 16;
constexpr int BN = 64;  // keys per tile

template <int NQB, int NW>
__global__ __launch_bounds__(64 * NW) void attn_bf16_flash(const unsigned short* __restrict__ q,
                                                           const unsigned short* __restrict__ k,
                                                           const unsigned short* __restrict__ v,
                                                           unsigned short* __restrict__ o, int Sq, int Sk, float c) {
  __shared__ __align__(16) unsigned short Ks[2][BN * KP];
  __shared__ __align__(16) unsigned short Vs[2][BN * VP];
  constexpr int NT = 64 * NW;
  constexpr int CPT = BN * 8 / NT;  // 16-byte chunks per thread per tile and tensor
  static_assert(CPT * NT == BN * 8, "tile must split evenly over the block");

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const size_t bh = blockIdx.y;
  const int q0 = (blockIdx.x * NW + w) * (16 * NQB);
  const unsigned short* qb = q + bh * (size_t)Sq * HD;
  const unsigned short* kb = k + bh * (size_t)Sk * HD;
  const unsigned short* vb = v + bh * (size_t)Sk * HD;

  // Q^T as B operands: lane owns query q0 + 16*i + col, dims 32*t + 8*grp .. +7.
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

  f32x4 O[4][NQB];
  float m[NQB], l[NQB];
#pragma unroll
  for (int i = 0; i < NQB; ++i) {
    m[i] = -INFINITY;
    l[i] = 0.0f;
#pragma unroll
    for (int db = 0; db < 4; ++db) O[db][i] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  uint4 kr[CPT], vr[CPT];
  auto gload = [&](int tile) {
#pragma unroll
    for (int ch = 0; ch < CPT; ++ch) {
      const int idx = tid + ch * NT, r = idx >> 3, cc = idx & 7;
      const int j = tile * BN + r;
      kr[ch] = make_uint4(0, 0, 0, 0);
      vr[ch] = make_uint4(0, 0, 0, 0);
      if (j < Sk) {
        kr[ch] = ld16(kb + (size_t)j * HD + cc * 8);
        vr[ch] = ld16(vb + (size_t)j * HD + cc * 8);
      }
    }
  };
  auto swrite = [&](int buf) {
#pragma unroll
    for (int ch = 0; ch < CPT; ++ch) {
      const int idx = tid + ch * NT, r = idx >> 3, cc = idx & 7;
      st16(&Ks[buf][r * KP + cc * 8], kr[ch]);
      st16(&Vs[buf][r * VP + cc * 8], vr[ch]);
    }
  };

  const int ntiles = (Sk + BN - 1) / BN;
  gload(0);
  swrite(0);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < ntiles) gload(t + 1);
    const unsigned short* Kt = Ks[buf];
    const unsigned short* Vt = Vs[buf];

    // S^T (64 keys x 16*NQB queries), four 16-key blocks.
    f32x4 S[4][NQB];
#pragma unroll
    for (int kb4 = 0; kb4 < 4; ++kb4) {
#pragma unroll
      for (int i = 0; i < NQB; ++i) S[kb4][i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(&Kt[(16 * kb4 + col) * KP + 32 * tt + 8 * grp]);
#pragma unroll
        for (int i = 0; i < NQB; ++i) S[kb4][i] = mfma_bf16(a, Qf[i][tt], S[kb4][i]);
      }
    }
    if ((t + 1) * BN > Sk) {  // ragged last tile: absent keys never enter max or sum
#pragma unroll
      for (int kb4 = 0; kb4 < 4; ++kb4)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool ok = t * BN + 16 * kb4 + 4 * grp + e < Sk;
#pragma unroll
          for (int i = 0; i < NQB; ++i) S[kb4][i][e] = ok ? S[kb4][i][e] : -INFINITY;
        }
    }

    // online softmax in the exp2 domain: p = 2^(s*c - m*c), c = scale*log2(e)
#pragma unroll
    for (int i = 0; i < NQB; ++i) {
      float mx = S[0][i][0];
#pragma unroll
      for (int kb4 = 0; kb4 < 4; ++kb4)
#pragma unroll
        for (int e = 0; e < 4; ++e) mx = fmaxf(mx, S[kb4][i][e]);
      mx = group4_max(mx);
      const float mnew = fmaxf(m[i], mx);
      const float alpha = fast_exp2((m[i] - mnew) * c);
      m[i] = mnew;
      const float mc = mnew * c;
      float ls = 0.0f;
#pragma unroll
      for (int kb4 = 0; kb4 < 4; ++kb4)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p = fast_exp2(__builtin_fmaf(S[kb4][i][e], c, -mc));
          S[kb4][i][e] = p;
          ls += p;
        }
      l[i] = __builtin_fmaf(l[i], alpha, ls);
#pragma unroll
      for (int db = 0; db < 4; ++db) O[db][i] *= alpha;
    }

    // O^T += V^T P^T over two 32-key steps.
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8 P[NQB];
#pragma unroll
      for (int i = 0; i < NQB; ++i) P[i] = pack_bf16(S[2 * ks][i], S[2 * ks + 1][i]);
      const int vrow = 32 * ks + 4 * grp + (col >> 2);
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int vcol = 16 * db + 4 * (col & 3);
        const i16x4 lo = lds_read_tr16(&Vt[vrow * VP + vcol]);
        const i16x4 hi = lds_read_tr16(&Vt[(vrow + 16) * VP + vcol]);
        const bf16x8 a = cat_bf16(lo, hi);
#pragma unroll
        for (int i = 0; i < NQB; ++i) O[db][i] = mfma_bf16(a, P[i], O[db][i]);
      }
    }

    if (t + 1 < ntiles) swrite(buf ^ 1);
    __syncthreads();
  }

  // epilogue: one division per output element row, after P.V
  unsigned short* ob = o + bh * (size_t)Sq * HD;
#pragma unroll
  for (int i = 0; i < NQB; ++i) {
    const float inv = 1.0f / group4_sum(l[i]);
    const int row = q0 + 16 * i + col;
    if (row < Sq) {
#pragma unroll
      for (int db = 0; db < 4; ++db)
        st8(ob + (size_t)row * HD + 16 * db + 4 * grp,
            pack4_bf16_bits(O[db][i][0] * inv, O[db][i][1] * inv, O[db][i][2] * inv, O[db][i][3] * inv));
    }
  }
}

// ---------------------------------------------------------------- bf16 cross (keys resident in LDS)
template <int NKB, int NQB, int NW>
__global__ __launch_bounds__(64 * NW) void xattn_bf16(const unsigned short* __restrict__ q,
                                                      const unsigned short* __restrict__ k,
                                                      const unsigned short* __restrict__ v,
                                                      unsigned short* __restrict__ o, int Sq, int Sk, float c) {
  static_assert(NKB % 2 == 0, "keys are consumed in 32-key steps");
  constexpr int NK = 16 * NKB;
  __shared__ __align__(16) unsigned short Ks[NK * KP];
  __shared__ __align__(16) unsigned short Vs[NK * VP];
  constexpr int NT = 64 * NW;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const size_t bh = blockIdx.y;
  const unsigned short* kb = k + bh * (size_t)Sk * HD;
  const unsigned short* vb = v + bh * (size_t)Sk * HD;

  // every key and value of this (b, h), rows past Sk zero (their scores are masked)
  for (int idx = tid; idx < NK * 8; idx += NT) {
    const int r = idx >> 3, cc = idx & 7;
    uint4 kk = make_uint4(0, 0, 0, 0), vv = kk;
    if (r < Sk) {
      kk = ld16(kb + (size_t)r * HD + cc * 8);
      vv = ld16(vb + (size_t)r * HD + cc * 8);
    }
    st16(&Ks[r * KP + cc * 8], kk);
    st16(&Vs[r * VP + cc * 8], vv);
  }
  __syncthreads();

  const int q0 = (blockIdx.x * NW + w) * (16 * NQB);
  if (q0 >= Sq) return;
  const unsigned short* qb = q + bh * (size_t)Sq * HD;
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

  f32x4 S[NKB][NQB];
#pragma unroll
  for (int kb_ = 0; kb_ < NKB; ++kb_) {
#pragma unroll
    for (int i = 0; i < NQB; ++i) S[kb_][i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(&Ks[(16 * kb_ + col) * KP + 32 * tt + 8 * grp]);
#pragma unroll
      for (int i = 0; i < NQB; ++i) S[kb_][i] = mfma_bf16(a, Qf[i][tt], S[kb_][i]);
    }
  }
  if (Sk < NK) {  // padded keys are set to -inf before the maximum is taken
#pragma unroll
    for (int kb_ = 0; kb_ < NKB; ++kb_)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool ok = 16 * kb_ + 4 * grp + e < Sk;
#pragma unroll
        for (int i = 0; i < NQB; ++i) S[kb_][i][e] = ok ? S[kb_][i][e] : -INFINITY;
      }
  }
  float l[NQB];
#pragma unroll
  for (int i = 0; i < NQB; ++i) {
    float mx = S[0][i][0];
#pragma unroll
    for (int kb_ = 0; kb_ < NKB; ++kb_)
#pragma unroll
      for (int e = 0; e < 4; ++e) mx = fmaxf(mx, S[kb_][i][e]);
    const float mc = group4_max(mx) * c;
    float ls = 0.0f;
#pragma unroll
    for (int kb_ = 0; kb_ < NKB; ++kb_)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p = fast_exp2(__builtin_fmaf(S[kb_][i][e], c, -mc));
        S[kb_][i][e] = p;
        ls += p;
      }
    l[i] = group4_sum(ls);
  }
  f32x4 O[4][NQB];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < NQB; ++i) O[db][i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < NKB / 2; ++ks) {
    bf16x8 P[NQB];
#pragma unroll
    for (int i = 0; i < NQB; ++i) P[i] = pack_bf16(S[2 * ks][i], S[2 * ks + 1][i]);
    const int vrow = 32 * ks + 4 * grp + (col >> 2);
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int vcol = 16 * db + 4 * (col & 3);
      const bf16x8 a = cat_bf16(lds_read_tr16(&Vs[vrow * VP + vcol]), lds_read_tr16(&Vs[(vrow + 16) * VP + vcol]));
#pragma unroll
      for (int i = 0; i < NQB; ++i) O[db][i] = mfma_bf16(a, P[i], O[db][i]);
    }
  }
  unsigned short* ob = o + bh * (size_t)Sq * HD;
#pragma unroll
  for (int i = 0; i < NQB; ++i) {
    const float inv = 1.0f / l[i];
    const int row = q0 + 16 * i + col;
    if (row < Sq) {
#pragma unroll
      for (int db = 0; db < 4; ++db)
        st8(ob + (size_t)row * HD + 16 * db + 4 * grp,
            pack4_bf16_bits(O[db][i][0] * inv, O[db][i][1] * inv, O[db][i][2] * inv, O[db][i][3] * inv));
    }
  }
}

// ---------------------------------------------------------------- launchers
hipError_t launch_attn_f32(const float* q, const float* k, const float* v, float* o, int B, int H, int Sq, int Sk,
                           float scale, hipStream_t s) {
  dim3 grid((Sq + F32_BQ - 1) / F32_BQ, B * H);
  hipLaunchKernelGGL(attn_f32_kernel, grid, dim3(F32_BQ), 0, s, q, k, v, o, Sq, Sk, scale);
  return hipGetLastError();
}

hipError_t launch_attn_bf16(const unsigned short* q, const unsigned short* k, const unsigned short* v,
                            unsigned short* o, int B, int H, int Sq, int Sk, float scale, hipStream_t s) {
  constexpr int NQB = 4, NW = 2;
  const float c = scale * LOG2E;
  dim3 grid((Sq + 16 * NQB * NW - 1) / (16 * NQB * NW), B * H);
  hipLaunchKernelGGL((attn_bf16_flash<NQB, NW>), grid, dim3(64 * NW), 0, s, q, k, v, o, Sq, Sk, c);
  return hipGetLastError();
}

template <int NKB, int NQB, int NW>
static hipError_t xlaunch(const unsigned short* q, const unsigned short* k, const unsigned short* v,
                          unsigned short* o, int B, int H, int Sq, int Sk, float c, hipStream_t s) {
  dim3 grid((Sq + 16 * NQB * NW - 1) / (16 * NQB * NW), B * H);
  hipLaunchKernelGGL((xattn_bf16<NKB, NQB, NW>), grid, dim3(64 * NW), 0, s, q, k, v, o, Sq, Sk, c);
  return hipGetLastError();
}

hipError_t launch_xattn_bf16(const unsigned short* q, const unsigned short* k, const unsigned short* v,
                             unsigned short* o, int B, int H, int Sq, int Sk, float scale, hipStream_t s) {
  const float c = scale * LOG2E;
  if (Sk <= 32) return xlaunch<2, 2, 2>(q, k, v, o, B, H, Sq, Sk, c, s);
  if (Sk <= 64) return xlaunch<4, 2, 2>(q, k, v, o, B, H, Sq, Sk, c, s);
  if (Sk <= 96) return xlaunch<6, 2, 2>(q, k, v, o, B, H, Sq, Sk, c, s);
  if (Sk <= 128) return xlaunch<8, 2, 2>(q, k, v, o, B, H, Sq, Sk, c, s);
  if (Sk <= 192) return xlaunch<12, 1, 4>(q, k, v, o, B, H, Sq, Sk, c, s);
  return xlaunch<16, 1, 4>(q, k, v, o, B, H, Sq, Sk, c, s);
}

}  // namespace ka
