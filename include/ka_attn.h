/*
 * ka_attn.h -- fused head-dim-64 attention for AMD MI355X (gfx950): the C ABI.
 *
 * Three operations, each one fused HIP kernel launch sequence enqueued on the
 * caller's stream:
 *
 *   ka_attn_fwd      dense scaled-dot-product attention (flash / online softmax)
 *   ka_xattn_fwd     cross-attention against a short key set held on chip
 *   ka_diffattn_fwd  differential attention with DyT and rotary embedding on Q/K,
 *                    banded (+-window keys) or full
 *   ka_diffattn_fwd_ex  the same with the Stable Audio 3 model's options: RMSNorm
 *                    on Q/K, rotary on 32 of the 64 dims, a V padding mask
 *
 * Common conventions
 *   - Pointers q, k, v, q1, k1, q2, k2, o, the parameter arrays and the
 *     workspace are DEVICE pointers owned by the caller.  The library never
 *     allocates, frees, synchronises or keeps a pointer after the call returns.
 *   - Every activation tensor is contiguous row-major [B][H][S][D] (D innermost);
 *     o has the layout of q (ka_diffattn_fwd_ex also takes strided views).  D is 64
 *     (ka_attn_fwd also takes 512).
 *   - Data types: KA_F32 (float32 in, float32 out, float32 arithmetic) or
 *     KA_BF16 (bfloat16 in, bfloat16 out; matrix products on bf16/fp16 MFMA with
 *     float32 accumulation; softmax, DyT, rotary embedding and the branch
 *     subtraction in float32).
 *   - Work is enqueued on `stream` and nothing else; the call returns without
 *     waiting.  Results are bitwise deterministic (no atomics).  Concurrent calls
 *     on different streams are safe: the library's only host state is a per-device
 *     cache of the CU count (atomic) and per-thread caches (the last HIP error,
 *     the last dense plan).
 *   - Shapes: B, H, Sq, Sk >= 1 and B*H*ceil(Sq/64) < 2^23 (every launch is a
 *     one-dimensional grid whose work-item count must fit 32 bits); otherwise
 *     KA_ERR_SHAPE.
 *   - Arguments are validated on the host before any HIP call; on failure
 *     nothing is enqueued and a status code is returned.  A failed launch
 *     returns KA_ERR_HIP and ka_last_hip_error() holds the hipError_t (per
 *     thread).  No C++ exception crosses this interface.
 *   - Inputs with NaN or Inf are outside the contract (they propagate).
 */
#ifndef KA_ATTN_H
#define KA_ATTN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KA_OK = 0,
  KA_ERR_NULL = 1,         /* a required pointer is NULL                                  */
  KA_ERR_SHAPE = 2,        /* a dimension < 1, Sq != Sk on the diff path, Sk above the
                              cross-attention limit, or a size overflowing 64 bits        */
  KA_ERR_UNSUPPORTED = 3,  /* a head dim or dtype this entry point does not take           */
  KA_ERR_PARAM = 4,        /* non-finite or non-positive scale, rope_base <= 1 or not
                              finite                                                      */
  KA_ERR_ALIGN = 5,        /* a tensor pointer is not 16-byte aligned                     */
  KA_ERR_ALIAS = 6,        /* o overlaps an input or the workspace                        */
  KA_ERR_WORKSPACE = 7,    /* workspace smaller than ka_diffattn_workspace_bytes()        */
  KA_ERR_HIP = 8           /* a HIP call failed; see ka_last_hip_error()                  */
} ka_status;

typedef enum { KA_F32 = 0, KA_BF16 = 1 } ka_dtype;

/* Largest key count ka_xattn_fwd holds on chip (longer key sets stream through): 512
 * keys and values at 304 bytes per key fill 152 KB of a CU's 160 KB of LDS. */
#define KA_XATTN_MAX_SK 512

/*
 * Dense scaled-dot-product attention, no mask.
 * Definition ("SDXL as a requirements inventory", s1.3, CrossAttention): for
 * every (b, h, i),
 *     o[b,h,i,:] = sum_j softmax_j(scale * <q[b,h,i,:], k[b,h,j,:]>) v[b,h,j,:]
 * with j over [0, Sk).  SDXL uses scale = 64^-1/2 = 0.125.
 *   q [B,H,Sq,D], k and v [B,H,Sk,D], o [B,H,Sq,D]; dtype KA_F32 or KA_BF16.
 *   Any B, H, Sq, Sk >= 1.  D = 64; or D = 512 with KA_BF16 (the SDXL VAE's
 *   single-head mid-block attention, 512 channels over 128 x 128 tokens,
 *   "SDXL as a requirements inventory" s1.5 and s5.10).
 */
ka_status ka_attn_fwd(ka_dtype dtype, const void* q, const void* k, const void* v, void* o, int B, int H, int Sq,
                      int Sk, int D, float scale, hipStream_t stream);

/*
 * Cross-attention: the same definition as ka_attn_fwd, for a key set of
 * conditioning tokens (SDXL's 77 text-context tokens, "SDXL as a requirements
 * inventory" s1.2 and s5.7; Stable Audio 3's 257 conditioning tokens, "401 ->
 * 163 ms..." appendix D2).  With 1 <= Sk <= KA_XATTN_MAX_SK all keys and values
 * of a (b, h) are held in LDS and re-read by every query tile, queries streaming
 * through (up to 128 keys one exact softmax pass, beyond that 64-key chunks with
 * an online softmax); longer key sets stream through LDS in tiles (the
 * ka_attn_fwd kernels).
 * Any Sk >= 1.
 *   dtype KA_BF16 (KA_F32 is accepted and routed to the fp32 kernel).
 */
ka_status ka_xattn_fwd(ka_dtype dtype, const void* q, const void* k, const void* v, void* o, int B, int H, int Sq,
                       int Sk, int D, float scale, hipStream_t stream);

/*
 * Differential attention with DyT and rotary embedding
 * ("401 -> 163 ms: Stable Audio 3 medium on one TPU v6e chip", s3, s5 and
 * appendix E1, E2, D4).  For every (b, h, p), with t in {q1, k1, q2, k2} and
 * set index 0..3 in that order:
 *   DyT:   x~ = gamma_t[d] * tanh(alpha_t * x[d]) + beta_t[d]            (fp32)
 *   RoPE:  rotate-half over all 64 dims at position p (token index):
 *          theta_i = p * rope_base^(-2i/64), i < 32,
 *          y[i]    = x~[i] cos theta_i - x~[i+32] sin theta_i,
 *          y[i+32] = x~[i+32] cos theta_i + x~[i] sin theta_i
 *   branch r = 1, 2:  O_r = sum_{j in W(p)} softmax_j(scale <q^_r[p], k^_r[j]>) v[j]
 *   output:           o[b,h,p,:] = O_1 - lambda[h] * O_2
 * W(p) = { j in [0, S) : |j - p| <= window } when window >= 0 (keys outside
 * [0, S) are absent, not zero), every j when window < 0.
 *   q1, k1, q2, k2, v, o: [B,H,S,D] bf16 (Sq must equal Sk = S); dtype KA_BF16.
 *   dyt_alpha [4], dyt_gamma [4][64], dyt_beta [4][64], lambda [H]: fp32 device.
 *   workspace: device scratch of at least ka_diffattn_workspace_bytes(B,H,S,D,
 *   window) bytes (may be NULL when that is 0); its contents are overwritten.
 * Precision: DyT, rotation, softmax and the subtraction in fp32; q^, k^ enter Q K^T as
 * fp16.  Banded path: weights bf16 against bf16 V.  Full and wide-window path: weights
 * and V as fp16, so V must lie within fp16 range, |v| <= 65504 (larger values saturate
 * to 65504; values below 2^-14 keep an absolute error under 2^-24).
 */
ka_status ka_diffattn_fwd(ka_dtype dtype, const void* q1, const void* k1, const void* q2, const void* k2,
                          const void* v, void* o, int B, int H, int Sq, int Sk, int D, float scale, int window,
                          const float* dyt_alpha, const float* dyt_gamma, const float* dyt_beta, float rope_base,
                          const float* lambda, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Q/K normaliser of ka_diffattn_fwd_ex. */
typedef enum { KA_QKNORM_DYT = 0, KA_QKNORM_RMS = 1 } ka_qknorm;

/* Element strides of a [B][H][S][64] bf16 view: element (b, h, s, d) sits at
 * base + b*batch + h*head + s*token + d.  The 64 dims of a token are contiguous. */
typedef struct {
  int64_t batch, head, token;
} ka_layout;

/*
 * Differential attention in the Stable Audio 3 model's own forms
 * ("401 -> 163 ms: Stable Audio 3 medium on one TPU v6e chip", appendix D1, D3,
 * D4, E1): ka_diffattn_fwd with three choices that call leaves fixed.
 *   qk_norm       KA_QKNORM_DYT: DyT with dyt_alpha, dyt_gamma, dyt_beta, as in
 *                 ka_diffattn_fwd (rms_weight is ignored and may be NULL).
 *                 KA_QKNORM_RMS: per-head RMSNorm in fp32,
 *                   x~[d] = rms_weight_t[d] * x[d] / sqrt(mean_d x[d]^2 + rms_eps),
 *                 rms_weight [4][64] fp32 device (sets q1, k1, q2, k2), rms_eps > 0
 *                 (the dyt_* pointers are ignored and may be NULL).
 *   rotary_dims   64: rotate-half over all dims, as ka_diffattn_fwd.
 *                 32: dims 0..31 only, dim i < 16 paired with dim i + 16 at
 *                 theta_i = p * rope_base^(-2i/32); dims 32..63 pass through.
 *   v_keep        NULL (every token kept), or [B][S] bytes on the device: a token
 *                 whose byte is 0 contributes a zero V row; its key stays in both
 *                 softmaxes (the model's padding mask, unlike key masking).
 *   layouts       NULL (every tensor contiguous [B][H][S][64]), or 6 views in the
 *                 order q1, k1, q2, k2, v, o, so that q1..v can be read straight out
 *                 of a fused projection (e.g. [B][S][5][H][64]: token = 5*H*64,
 *                 head = 64) and o written merged ([B][S][H][64]), with no transposes
 *                 ("401 -> 163 ms...", appendix E1 "No transposes", D3).  Each stride
 *                 is a non-negative multiple of 8, token >= 64, and one (b, h) slice
 *                 spans under 2^31 bytes (else KA_ERR_SHAPE); o's rows must not
 *                 overlap each other (KA_ERR_SHAPE) nor any input's extent, the span
 *                 from its base to its last row (KA_ERR_ALIAS).  Inputs may share memory.
 * Everything else -- shapes, dtype, window, lambda, workspace, errors -- is as for
 * ka_diffattn_fwd; rotary_dims other than 32 or 64, or a non-positive or
 * non-finite rms_eps, give KA_ERR_PARAM; an unknown qk_norm KA_ERR_UNSUPPORTED.
 */
ka_status ka_diffattn_fwd_ex(ka_dtype dtype, const void* q1, const void* k1, const void* q2, const void* k2,
                             const void* v, void* o, int B, int H, int Sq, int Sk, int D, float scale, int window,
                             ka_qknorm qk_norm, const float* dyt_alpha, const float* dyt_gamma,
                             const float* dyt_beta, const float* rms_weight, float rms_eps, int rotary_dims,
                             float rope_base, const float* lambda, const uint8_t* v_keep,
                             const ka_layout* layouts, void* workspace, size_t workspace_bytes,
                             hipStream_t stream);

/* Size of the device scratch array behind ka_diffattn_fwd_noalloc (one copy per GPU). */
#define KA_STATIC_WORKSPACE_BYTES ((size_t)32 << 20)

/*
 * ka_diffattn_fwd_ex without a workspace argument, for callers that cannot allocate
 * device memory (code under stream capture, tight serving loops, harnesses that forbid
 * allocation).  The full path's scratch (ka_diffattn_workspace_bytes of the shape) comes
 * from a file-scope device array of KA_STATIC_WORKSPACE_BYTES that each GPU holds for the
 * life of the process; the call itself allocates and frees nothing.  Shapes needing more
 * return KA_ERR_WORKSPACE (before any HIP call): 32 MiB covers B*H*S up to 87,381 rows
 * (the 1422-token DiT shape with 16 heads needs 8.7 MB).  Calls on one GPU share the array:
 * calls that overlap in time on one GPU (different streams, or different threads without
 * ordering) race on it and give undefined results; calls ordered on one stream are safe.
 * The banded path needs no scratch.  Everything else is as for ka_diffattn_fwd_ex; the
 * first call on a device looks up the array's address (a HIP call; a failure returns
 * KA_ERR_HIP).
 */
ka_status ka_diffattn_fwd_noalloc(ka_dtype dtype, const void* q1, const void* k1, const void* q2, const void* k2,
                                  const void* v, void* o, int B, int H, int Sq, int Sk, int D, float scale,
                                  int window, ka_qknorm qk_norm, const float* dyt_alpha, const float* dyt_gamma,
                                  const float* dyt_beta, const float* rms_weight, float rms_eps, int rotary_dims,
                                  float rope_base, const float* lambda, const uint8_t* v_keep,
                                  const ka_layout* layouts, hipStream_t stream);

/* Workspace bytes ka_diffattn_fwd and ka_diffattn_fwd_ex need for this shape: 0 for
 * the banded path; for the full (and wide-window) path three fp16 planes of B*H*S*64:
 * the prepared keys k1^ and k2^, and V converted to fp16 (rows of tokens flagged out by
 * v_keep zeroed).  Returns 0 for invalid shapes as well; the call then reports the
 * error. */
size_t ka_diffattn_workspace_bytes(int B, int H, int S, int D, int window);

/* Name of the kernel (and query layout) ka_attn_fwd launches for this shape on the
 * current device, e.g. "attn_bf16_quad 3+2", "attn_bf16_duo 3+3", "attn_bf16_pipe",
 * "attn_f32", "attn512_pair"; NULL for a shape or dtype ka_attn_fwd rejects.  A static
 * string.  For tuning and for checks that every layout computes the same result. */
const char* ka_attn_kernel_name(ka_dtype dtype, int B, int H, int Sq, int Sk, int D);

/* Static description of a status code. */
const char* ka_status_string(ka_status status);

/* hipError_t of the last KA_ERR_HIP returned on the calling thread (0 if none). */
int ka_last_hip_error(void);

/* Library version as "major.minor.patch". */
const char* ka_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KA_ATTN_H */
