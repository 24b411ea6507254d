/*
 * ka_oracle.c -- plain, slow, fp64 CPU oracle for fused head-dim-64 attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the library under head_attention_flash_amd/
 * links, includes or calls this file; only tests/, the smoke check in
 * __graft_entry__.py and the cpu_baseline leg of bench.py use it.  It shares no
 * code, header, table or constant with the HIP path.
 *
 * Every input arrives as float64 holding the exact stored value (a bf16 or fp32
 * element widens to double without rounding); parameters arrive as the float32
 * values the caller passes, widened.  Nothing is rounded inside: each output is
 * the plain definition evaluated in double precision.
 *
 * Sources (the pages, by title and section):
 *  - "SDXL as a requirements inventory", s1.3 (CrossAttention): per head,
 *    O = softmax(q k^T * 64^-1/2) v on tensors shaped [B*heads, L, 64]; no mask.
 *  - same page, s2.1: attention work is B*heads*Lq*Lkv*D multiply-adds for the
 *    scores and the same again for the weighted sum.
 *  - "401 -> 163 ms: Stable Audio 3 medium on one TPU v6e chip", s3 and appendix
 *    E1: the decoder's differential attention normalises q and k (DyT), applies
 *    rotary embedding by rotate-half, runs two softmax branches over a band of
 *    +-17 keys around each query (masked by nominal position, so keys past either
 *    end of the sequence are absent, not zero), and subtracts the second branch
 *    from the first; both branches weight the same V.  Appendix E2: rows of V
 *    outside [0, S) must not contribute.  Section 5 / appendix D4: the same
 *    computation without the band (every key visible).
 *  - The DyT formula gamma*tanh(alpha*x)+beta, the rotary width (all 64 dims,
 *    pairs (i, i+32)), base 10000, and the per-head weight lambda on branch 2 are
 *    not defined on the pages; they are the readings this library adopts.
 *  - The Stable Audio 3 model's own forms (same page, appendix D1, D3, D4, E1):
 *    per-head RMSNorm on q and k in place of DyT; rotary embedding on part of
 *    the head only (rotate-half pairs d with d+16, the other dims pass through
 *    with cos 1, sin 0: a rotary width of 32); and a padding mask that zeroes V
 *    for padded tokens while their keys stay in the softmax.  RMSNorm's formula
 *    (x / sqrt(mean x^2 + eps), times a learned weight per dim) and eps are not
 *    on the pages; the standard definition is the reading taken.
 *
 * Softmax is two-pass (max, then exp and sum), the textbook stable form; the
 * online (running-max) form used by the GPU reaches the same value in exact
 * arithmetic.
 *
 * Parity pins: every function here is pinned by the CPU tests (closed forms,
 * invariants, special cases, a long-double brute force and torch's float64 SDPA).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORA_OK 0
#define ORA_EBADARG 1
#define ORA_ENOMEM 2

/* ---------------------------------------------------------------- building blocks */

/* DyT of one head row: y[d] = gamma[d] * tanh(alpha * x[d]) + beta[d]. */
void ora_dyt_row(const double* x, int D, double alpha, const double* gamma, const double* beta, double* y) {
  for (int d = 0; d < D; ++d) y[d] = gamma[d] * tanh(alpha * x[d]) + beta[d];
}

/* Rotary embedding of one head row at token position p, rotate-half convention
 * over all D dims: dim i pairs with dim i + D/2, angle theta_i = p * base^(-2i/D),
 *   y[i]       = x[i] cos(theta_i) - x[i+D/2] sin(theta_i)
 *   y[i+D/2]   = x[i+D/2] cos(theta_i) + x[i] sin(theta_i).            */
void ora_rope_row(const double* x, int D, long p, double base, double* y) {
  int half = D / 2;
  for (int i = 0; i < half; ++i) {
    double theta = (double)p * pow(base, -2.0 * (double)i / (double)D);
    double c = cos(theta), s = sin(theta);
    y[i] = x[i] * c - x[i + half] * s;
    y[i + half] = x[i + half] * c + x[i] * s;
  }
}

/* RMSNorm of one head row: y[d] = w[d] * x[d] / sqrt(mean_d x[d]^2 + eps). */
void ora_rmsnorm_row(const double* x, int D, double eps, const double* w, double* y) {
  double ss = 0.0;
  for (int d = 0; d < D; ++d) ss += x[d] * x[d];
  const double inv = 1.0 / sqrt(ss / (double)D + eps);
  for (int d = 0; d < D; ++d) y[d] = w[d] * (x[d] * inv);
}

/* Rotary embedding on the first `rot` dims of a head row (rot even, 2 <= rot <= D),
 * rotate-half within them: dim i < rot/2 pairs with dim i + rot/2 at angle
 * theta_i = p * base^(-2i/rot); dims rot .. D-1 pass through unchanged.          */
void ora_rope_row_partial(const double* x, int D, int rot, long p, double base, double* y) {
  int h = rot / 2;
  for (int d = rot; d < D; ++d) y[d] = x[d];
  for (int i = 0; i < h; ++i) {
    double th = (double)p * pow(base, -2.0 * (double)i / (double)rot);
    double c = cos(th), s = sin(th);
    y[i] = x[i] * c - x[h + i] * s;
    y[h + i] = x[h + i] * c + x[i] * s;
  }
}

/* One output row of softmax attention over an explicit key set.
 * q: [D]; keys / vals: row pointers (nk of them); out: [D].
 *   s_j = scale * <q, k_j>;  m = max_j s_j;  e_j = exp(s_j - m);  out = sum_j e_j v_j / sum_j e_j */
static void attend_row(const double* q, const double* const* keys, const double* const* vals, int nk, int D,
                       double scale, double* s, double* out) {
  double m = -INFINITY;
  for (int j = 0; j < nk; ++j) {
    double acc = 0.0;
    for (int d = 0; d < D; ++d) acc += q[d] * keys[j][d];
    s[j] = scale * acc;
    if (s[j] > m) m = s[j];
  }
  double z = 0.0;
  for (int j = 0; j < nk; ++j) {
    s[j] = exp(s[j] - m);
    z += s[j];
  }
  for (int d = 0; d < D; ++d) out[d] = 0.0;
  for (int j = 0; j < nk; ++j)
    for (int d = 0; d < D; ++d) out[d] += s[j] * vals[j][d];
  for (int d = 0; d < D; ++d) out[d] /= z;
}

/* ---------------------------------------------------------------- dense / cross attention */

/* Scaled-dot-product attention, no mask, for a list of output rows.
 * q [B,H,Sq,D], k/v [B,H,Sk,D], out [B,H,Sq,D]; rows == NULL means every row,
 * else rows[r] is the flat index (b*H + h)*Sq + i of a row to compute (only those
 * rows of out are written).  Dense self-attention and cross-attention are the
 * same definition; they differ only in Sk.                                          */
int ora_attn(const double* q, const double* k, const double* v, double* out, int B, int H, int Sq, int Sk, int D,
             double scale, const int64_t* rows, int64_t nrows) {
  if (!q || !k || !v || !out || B < 1 || H < 1 || Sq < 1 || Sk < 1 || D < 1) return ORA_EBADARG;
  int64_t total = rows ? nrows : (int64_t)B * H * Sq;
  int err = 0;
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * Sk);
    const double** kr = (const double**)malloc(sizeof(double*) * Sk);
    const double** vr = (const double**)malloc(sizeof(double*) * Sk);
    if (!s || !kr || !vr) {
#pragma omp atomic write
      err = ORA_ENOMEM;
    } else {
#pragma omp for schedule(dynamic, 16)
      for (int64_t r = 0; r < total; ++r) {
        int64_t flat = rows ? rows[r] : r;
        int64_t bh = flat / Sq;
        const double* kb = k + bh * (int64_t)Sk * D;
        const double* vb = v + bh * (int64_t)Sk * D;
        for (int j = 0; j < Sk; ++j) {
          kr[j] = kb + (int64_t)j * D;
          vr[j] = vb + (int64_t)j * D;
        }
        attend_row(q + flat * D, kr, vr, Sk, D, scale, s, out + flat * D);
      }
    }
    free(s);
    free((void*)kr);
    free((void*)vr);
  }
  return err;
}

/* ---------------------------------------------------------------- differential attention */

/* The key set of query p: all j in [0, S) with |j - p| <= window, or every j when
 * window < 0.  Returns the first key and the count.                                */
static void window_of(long p, int S, int window, int* j0, int* nk) {
  if (window < 0) {
    *j0 = 0;
    *nk = S;
    return;
  }
  long lo = p - window, hi = p + window;
  if (lo < 0) lo = 0;
  if (hi > S - 1) hi = S - 1;
  *j0 = (int)lo;
  *nk = (int)(hi - lo + 1);
}

#define ORA_NORM_DYT 0
#define ORA_NORM_RMS 1

/* How the q/k rows are prepared: the normaliser (DyT with alpha, gamma, beta, or
 * RMSNorm with eps and weight w) and the rotary width rot (D: every dim). */
typedef struct {
  int norm;
  double eps;
  int rot;
} prep_mode;

/* Prepare (normalise, then rotate) every row of one [S, D] slice with parameter set t. */
static void prep_slice(const double* x, int S, int D, prep_mode m, double alpha, const double* gamma,
                       const double* beta, const double* w, double base, double* tmp, double* y) {
  for (int p = 0; p < S; ++p) {
    if (m.norm == ORA_NORM_RMS)
      ora_rmsnorm_row(x + (int64_t)p * D, D, m.eps, w, tmp);
    else
      ora_dyt_row(x + (int64_t)p * D, D, alpha, gamma, beta, tmp);
    if (m.rot == D)
      ora_rope_row(tmp, D, p, base, y + (int64_t)p * D);
    else
      ora_rope_row_partial(tmp, D, m.rot, p, base, y + (int64_t)p * D);
  }
}

/* Differential attention, general form.  Inputs q1,k1,q2,k2,v [B,H,S,D]; out
 * [B,H,S,D].  Normaliser: norm = ORA_NORM_DYT with alpha[4], gamma[4*D], beta[4*D],
 * or ORA_NORM_RMS with eps and rms_w[4*D] (set t = 0:q1, 1:k1, 2:q2, 3:k2); rotary
 * width rot (D, or an even width below it); lam[H]; v_keep [B*S] or NULL (all kept).
 * For each (b, h, p):
 *   qt = RoPE_p(Norm_t(q_t[p])), kt = RoPE_j(Norm_t(k_t[j]))         (t = q1,k1 / q2,k2)
 *   O_r = softmax_{j in W(p)}(scale <q_r, k_r,j>) . V'[j]              (r = 1, 2)
 *   V'[j] = V[j] if v_keep[b*S + j] != 0, else 0 (key j stays in the softmax)
 *   out = O_1 - lam[h] * O_2
 * rows as in ora_attn (flat index (b*H + h)*S + p).                                  */
int ora_diffattn_ex(const double* q1, const double* k1, const double* q2, const double* k2, const double* v,
                    double* out, int B, int H, int S, int D, double scale, int window, int norm, const double* alpha,
                    const double* gamma, const double* beta, double eps, const double* rms_w, int rot, double base,
                    const double* lam, const unsigned char* v_keep, const int64_t* rows, int64_t nrows) {
  if (!q1 || !k1 || !q2 || !k2 || !v || !out || !lam) return ORA_EBADARG;
  if (norm == ORA_NORM_DYT && (!alpha || !gamma || !beta)) return ORA_EBADARG;
  if (norm == ORA_NORM_RMS && (!rms_w || !(eps >= 0.0))) return ORA_EBADARG;
  if (norm != ORA_NORM_DYT && norm != ORA_NORM_RMS) return ORA_EBADARG;
  if (B < 1 || H < 1 || S < 1 || D < 2 || (D % 2) || rot < 2 || rot > D || (rot % 2)) return ORA_EBADARG;
  const double* src[4] = {q1, k1, q2, k2};
  const prep_mode mode = {norm, eps, rot};
  int64_t plane = (int64_t)S * D;
  int err = 0;
  double* zero_row = (double*)calloc((size_t)D, sizeof(double));
  if (!zero_row) return ORA_ENOMEM;
  /* one (b, h) slice at a time: prepare all four tensors of the slice, then attend
   * the requested rows of that slice. */
  double* prep = (double*)malloc(sizeof(double) * 4 * plane);
  if (!prep) {
    free(zero_row);
    return ORA_ENOMEM;
  }
  for (int64_t bh = 0; bh < (int64_t)B * H && !err; ++bh) {
    int h = (int)(bh % H);
    /* which rows of this slice are wanted */
    int any = rows ? 0 : 1;
    if (rows)
      for (int64_t r = 0; r < nrows; ++r)
        if (rows[r] / S == bh) { any = 1; break; }
    if (!any) continue;
#pragma omp parallel for schedule(static)
    for (int t = 0; t < 4; ++t) {
      double* tmp = (double*)malloc(sizeof(double) * D);
      if (!tmp) {
#pragma omp atomic write
        err = ORA_ENOMEM;
        continue;
      }
      const int dyt = norm == ORA_NORM_DYT;
      prep_slice(src[t] + bh * plane, S, D, mode, dyt ? alpha[t] : 0.0, dyt ? gamma + (int64_t)t * D : NULL,
                 dyt ? beta + (int64_t)t * D : NULL, dyt ? NULL : rms_w + (int64_t)t * D, base, tmp,
                 prep + (int64_t)t * plane);
      free(tmp);
    }
    if (err) break;
    const double* qh1 = prep + 0 * plane;
    const double* kh1 = prep + 1 * plane;
    const double* qh2 = prep + 2 * plane;
    const double* kh2 = prep + 3 * plane;
    const double* vb = v + bh * plane;
    const unsigned char* keep = v_keep ? v_keep + (bh / H) * (int64_t)S : NULL;
    int64_t nr = rows ? nrows : S;
#pragma omp parallel
    {
      double* s = (double*)malloc(sizeof(double) * S);
      const double** kr1 = (const double**)malloc(sizeof(double*) * S);
      const double** kr2 = (const double**)malloc(sizeof(double*) * S);
      const double** vr = (const double**)malloc(sizeof(double*) * S);
      double* o1 = (double*)malloc(sizeof(double) * D);
      double* o2 = (double*)malloc(sizeof(double) * D);
      if (!s || !kr1 || !kr2 || !vr || !o1 || !o2) {
#pragma omp atomic write
        err = ORA_ENOMEM;
      } else {
#pragma omp for schedule(dynamic, 16)
        for (int64_t r = 0; r < nr; ++r) {
          int64_t flat = rows ? rows[r] : bh * S + r;
          if (flat / S != bh) continue;
          long p = (long)(flat % S);
          int j0, nk;
          window_of(p, S, window, &j0, &nk);
          for (int j = 0; j < nk; ++j) {
            kr1[j] = kh1 + (int64_t)(j0 + j) * D;
            kr2[j] = kh2 + (int64_t)(j0 + j) * D;
            vr[j] = (keep && !keep[j0 + j]) ? zero_row : vb + (int64_t)(j0 + j) * D;
          }
          attend_row(qh1 + p * D, kr1, vr, nk, D, scale, s, o1);
          attend_row(qh2 + p * D, kr2, vr, nk, D, scale, s, o2);
          for (int d = 0; d < D; ++d) out[flat * D + d] = o1[d] - lam[h] * o2[d];
        }
      }
      free(s);
      free((void*)kr1);
      free((void*)kr2);
      free((void*)vr);
      free(o1);
      free(o2);
    }
  }
  free(prep);
  free(zero_row);
  return err;
}

/* Differential attention with DyT and rotary embedding over every dim, no V mask. */
int ora_diffattn(const double* q1, const double* k1, const double* q2, const double* k2, const double* v,
                 double* out, int B, int H, int S, int D, double scale, int window, const double* alpha,
                 const double* gamma, const double* beta, double base, const double* lam, const int64_t* rows,
                 int64_t nrows) {
  if (!alpha || !gamma || !beta) return ORA_EBADARG;
  return ora_diffattn_ex(q1, k1, q2, k2, v, out, B, H, S, D, scale, window, ORA_NORM_DYT, alpha, gamma, beta, 0.0,
                         NULL, D, base, lam, NULL, rows, nrows);
}

/* Number of OpenMP threads the oracle will use (reported beside its timings). */
int ora_num_threads(void) {
#ifdef _OPENMP
  extern int omp_get_max_threads(void);
  return omp_get_max_threads();
#else
  return 1;
#endif
}
