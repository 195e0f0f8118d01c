/*
 * moe_oracle.c -- TEST INFRASTRUCTURE, not part of the product.
 *
 * A plain, slow, obviously-correct CPU statement of the forward pass of one
 * Mixture-of-Experts FFN layer, in double precision, written from the pages'
 * description of the method. Only the test-suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load it. It shares no code, header,
 * table or helper with the HIP library and includes nothing from it.
 *
 * Sources (cited by page title and section):
 *  [DSC]  "DeepSpeed MoE and Model Compression" (shaojiemike.top),
 *         section "DeepSpeed-MoE" (the equation p(x)=softmax(W_r x),
 *         y = sum over TopK(p,k) of p_e(x) E_e(x), and the pipeline block:
 *         router -> topk -> pack_by_expert(capacity) -> experts -> combine
 *         with gates, plus a load-balance loss).
 *  [DvS]  "DeepSpeed-MoE vs Switch Transformer" (hncyxsy.com), sections
 *         "router computation" (logits = x W_r, p = softmax(logits)),
 *         "Top-1 routing decision", "expert capacity overflow" (capacity =
 *         tokens / experts x capacity_factor; an overflowing token skips the
 *         expert FFN and reaches the next layer through the residual),
 *         "PR-MoE residual example".
 *  [SRV]  "MoE survey, pruning and quantization notes" (ken1301225.github.io),
 *         sec. 1.1.1.1 (TopK after softmax needs renormalisation),
 *         sec. 1.1.2.1 (an expert is a two-layer FFN; MoE(x)=sum w_i M_i(x)),
 *         sec. 1.1.4.1 (Switch load-balance loss alpha*N*sum f_i Q_i),
 *         sec. 1.2.1 (bf16 is the top half of an fp32),
 *         sec. 1.2.2 (symmetric quantization: r_hat = s*q).
 *  [SRV2] the same survey notes, sec. 1.1.1.1 (linear gating with TopK and a
 *         noise term R_noise that encourages exploration), sec. 1.1.1.2
 *         (cosine-similarity gating with a learnable projection, expert
 *         embeddings and a temperature tau), sec. 1.1.4.1 (Importance and
 *         Load losses: w * CoV(.)^2 of per-expert sums), sec. 1.1.4.2 (TopP
 *         expert selection by accumulated score).
 *  [DSN]  "DeepSpeed-MoE: Advancing Mixture-of-Experts Inference and Training
 *         to Power Next-Generation AI Scale" (unpurerationalist.github.io
 *         notes), sec. 3.1 (Residual-MoE: fixed dense MLP plus one top-1
 *         expert as a residual correction), sec. 4.4 (cumsum mapping table).
 *
 * Readings where the pages are silent are listed in the design doc; the ones
 * that shape this file are restated next to the code they affect.
 *
 * Element formats accepted for x and weights (exactly converted to double):
 *   OR_F32  : IEEE binary32
 *   OR_BF16 : bfloat16 bit patterns (uint16), the upper half of a binary32
 *   OR_I8   : signed 8-bit codes, with one float32 scale per 128 consecutive
 *             input-dimension elements of each output row (symmetric int8)
 *   OR_F64  : IEEE binary64 (lets the finite-difference checks of the
 *             backward perturb inputs by tiny steps)
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_F32 = 0, OR_BF16 = 1, OR_I8 = 2, OR_F64 = 3 };
enum { OR_DROP_TOKEN_ORDER = 0, OR_DROP_GATE_PRIORITY = 1 };

#define OR_GROUP 128

/* value of element i of an array in one of the formats above */
static double elem(const void *p, int fmt, int64_t i) {
  if (fmt == OR_F32) return (double)((const float *)p)[i];
  if (fmt == OR_F64) return ((const double *)p)[i];
  if (fmt == OR_BF16) {
    uint32_t u = (uint32_t)((const uint16_t *)p)[i] << 16; /* [SRV] 1.2.1 */
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
  }
  return (double)((const int8_t *)p)[i];
}

/* weight element (n, i) of an [N, K] row-major matrix; int8 codes are
 * dequantised as scale * code with the scale of group i / 128 of row n
 * ([SRV] 1.2.2, symmetric form). */
static double weight(const void *w, int fmt, const float *scale, int64_t N,
                     int64_t K, int64_t n, int64_t i) {
  (void)N;
  double v = elem(w, fmt, n * K + i);
  if (fmt == OR_I8) v *= (double)scale[n * (K / OR_GROUP) + i / OR_GROUP];
  return v;
}

/* exact (erf) GELU; the configurations name GELU as the FFN activation */
static double gelu(double z) { return 0.5 * z * (1.0 + erf(z / sqrt(2.0))); }

/* ------------------------------------------------------------------------
 * Capacity.  [DvS] "expert capacity overflow": capacity = tokens per batch /
 * number of experts x capacity_factor.  Reading: with top-k routing there
 * are k*T assignments, so C = ceil(k*T*cf/E); a positive override replaces
 * it; C is clamped to T (no expert can receive more than T assignments
 * because a token's k experts are distinct, so the clamp changes nothing).
 * ---------------------------------------------------------------------- */
int64_t oracle_capacity(int64_t T, int64_t E, int64_t k, double cf,
                        int64_t override_c) {
  int64_t c;
  if (override_c > 0)
    c = override_c;
  else
    c = (int64_t)ceil((double)k * (double)T * cf / (double)E);
  if (c > T) c = T;
  if (c < 0) c = 0;
  return c;
}

/* ------------------------------------------------------------------------
 * Router.  [DSC] eq. p(x) = softmax(W_r x); [DvS] "router computation".
 * logits[t,e] = sum_i x[t,i] W_r[e,i] (+ b[e]); p = softmax over e.
 * Top-k: the k largest probabilities, in descending order, ties to the lower
 * expert index.  Softmax is strictly increasing in the logit, so ranking by
 * logits ranks by probability.
 * Gates: k = 1 -> the chosen expert's full-softmax probability ([DSC] eq.);
 * k >= 2 with normalize -> p_j / sum of the k chosen p ([SRV] 1.1.1.1),
 * without normalize -> p_j.
 * ---------------------------------------------------------------------- */
int oracle_route(int64_t T, int64_t d, int64_t E, int64_t k, int normalize,
                 const void *x, int x_fmt, const void *wr, int wr_fmt,
                 const float *bias, double *logits, double *probs,
                 int32_t *ids, double *gates) {
  if (k < 1 || k > E) return -1;
#pragma omp parallel for schedule(dynamic, 4)
  for (int64_t t = 0; t < T; t++) {
    double *l = logits + t * E, *p = probs + t * E;
    for (int64_t e = 0; e < E; e++) {
      double s = 0.0;
      for (int64_t i = 0; i < d; i++)
        s += elem(x, x_fmt, t * d + i) * elem(wr, wr_fmt, e * d + i);
      if (bias) s += (double)bias[e];
      l[e] = s;
    }
    double m = l[0];
    for (int64_t e = 1; e < E; e++)
      if (l[e] > m) m = l[e];
    double z = 0.0;
    for (int64_t e = 0; e < E; e++) {
      p[e] = exp(l[e] - m);
      z += p[e];
    }
    for (int64_t e = 0; e < E; e++) p[e] /= z;

    /* selection: repeatedly take the best not-yet-chosen expert under the
     * order (larger logit first, then smaller index) */
    int32_t *sel = ids + t * k;
    for (int64_t j = 0; j < k; j++) {
      int64_t best = -1;
      for (int64_t e = 0; e < E; e++) {
        int taken = 0;
        for (int64_t q = 0; q < j; q++)
          if (sel[q] == e) taken = 1;
        if (taken) continue;
        if (best < 0 || l[e] > l[best]) best = e; /* strict: keeps lower index on ties */
      }
      sel[j] = (int32_t)best;
    }
    double *g = gates + t * k;
    double den = 0.0;
    for (int64_t j = 0; j < k; j++) den += p[sel[j]];
    for (int64_t j = 0; j < k; j++)
      g[j] = (k >= 2 && normalize) ? p[sel[j]] / den : p[sel[j]];
  }
  return 0;
}

/* ------------------------------------------------------------------------
 * Switch load-balance loss.  [SRV] 1.1.4.1:
 *   f_i = (1/T) #{tokens whose argmax expert is i}
 *   Q_i = (1/T) sum over tokens of the router probability of i
 *   loss = alpha * N * sum_i f_i Q_i,   N = number of experts.
 * Readings: the argmax is the first-ranked choice ids[t,0] (also for k=2);
 * f counts routing decisions before any capacity drop; Q uses the full
 * softmax (bias included).  T = 0 gives loss 0 (both sums are empty).
 * f and Q are written out when the pointers are non-NULL.
 * ---------------------------------------------------------------------- */
double oracle_aux_loss(int64_t T, int64_t E, int64_t k, const int32_t *ids,
                       const double *probs, double alpha, double *f_out,
                       double *q_out) {
  double *f = (double *)calloc((size_t)(E > 0 ? E : 1), sizeof(double));
  double *q = (double *)calloc((size_t)(E > 0 ? E : 1), sizeof(double));
  for (int64_t t = 0; t < T; t++) {
    f[ids[t * k]] += 1.0;
    for (int64_t e = 0; e < E; e++) q[e] += probs[t * E + e];
  }
  double loss = 0.0;
  if (T > 0) {
    for (int64_t e = 0; e < E; e++) {
      f[e] /= (double)T;
      q[e] /= (double)T;
      loss += f[e] * q[e];
    }
    loss *= alpha * (double)E;
  }
  if (f_out) memcpy(f_out, f, (size_t)E * sizeof(double));
  if (q_out) memcpy(q_out, q, (size_t)E * sizeof(double));
  free(f);
  free(q);
  return loss;
}

/* ------------------------------------------------------------------------
 * Dispatch into the expert-major capacity buffer.  [DSC] pack_by_expert with
 * a capacity; [DvS] overflow tokens skip the expert; [DSN] 4.4 builds the
 * token-to-expert mapping from a cumulative sum over tokens.
 *
 * OR_DROP_TOKEN_ORDER (the contract): an expert takes its assignments in
 * token order; the n-th one (counting from 0) gets slot n and is kept iff
 * n < C.  A token's k experts are distinct, so token order is a total order
 * within one expert.
 * OR_DROP_GATE_PRIORITY ([DvS] capacity example): an expert keeps its C
 * assignments with the largest gate (ties to the earlier token); the slot is
 * the rank in that order.
 * Outputs: slots[t,j] (-1 when dropped), drop[t,j] (1 when dropped),
 * load[e] = assignments received, kept[e] = min(load[e], C).  Entries whose
 * id is not an expert are no assignment (slot -1, drop 0).
 * ---------------------------------------------------------------------- */
int oracle_dispatch(int64_t T, int64_t E, int64_t k, int64_t C,
                    const int32_t *ids, const double *gates, int policy,
                    int32_t *slots, uint8_t *drop, int32_t *load,
                    int32_t *kept) {
  if (policy == OR_DROP_GATE_PRIORITY && !gates) return -1;
  /* an id outside 0..E-1 (a TopP token that chose fewer than k experts)
   * is no assignment: slot -1, not dropped, counted nowhere */
  for (int64_t a = 0; a < T * k; a++) {
    slots[a] = -1;
    drop[a] = 0;
  }
  for (int64_t e = 0; e < E; e++) {
    int64_t n = 0;
    for (int64_t t = 0; t < T; t++)
      for (int64_t j = 0; j < k; j++) {
        if (ids[t * k + j] != e) continue;
        int64_t rank;
        if (policy == OR_DROP_TOKEN_ORDER) {
          rank = n;
        } else {
          /* number of this expert's assignments that come before (t,j) */
          rank = 0;
          double g = gates[t * k + j];
          for (int64_t u = 0; u < T; u++)
            for (int64_t i = 0; i < k; i++) {
              if (ids[u * k + i] != e) continue;
              double h = gates[u * k + i];
              if (h > g || (h == g && u < t)) rank++;
            }
        }
        n++;
        if (rank < C) {
          slots[t * k + j] = (int32_t)rank;
          drop[t * k + j] = 0;
        } else {
          slots[t * k + j] = -1;
          drop[t * k + j] = 1;
        }
      }
    load[e] = (int32_t)n;
    kept[e] = (int32_t)(n < C ? n : C);
  }
  return 0;
}

/* ------------------------------------------------------------------------
 * Two-layer GELU FFN on a list of rows with one weight pair.
 * [SRV] 1.1.2.1: an expert is a two-layer feed-forward network; the
 * configurations name GELU and no biases.  Weights are [out, in] row-major:
 * W1 [F, D], W2 [D, F].   h = GELU(W1 x) (F values);  out = W2 h (D values).
 * The same function states PR-MoE's fixed dense MLP ([DSN] 3.1).
 * rows: n x D in x_fmt; out: n x D doubles; h_out (optional): n x F.
 * ---------------------------------------------------------------------- */
/* one row: h = GELU(W1 x), out = W2 h; h is caller scratch of F doubles */
static void ffn_one_row(int64_t D, int64_t F, const void *xr, int x_fmt,
                        int64_t row, const void *w1, const void *w2, int w_fmt,
                        const float *s1, const float *s2, double *h,
                        double *out) {
  for (int64_t f = 0; f < F; f++) {
    double s = 0.0;
    for (int64_t i = 0; i < D; i++)
      s += weight(w1, w_fmt, s1, F, D, f, i) * elem(xr, x_fmt, row * D + i);
    h[f] = gelu(s);
  }
  for (int64_t o = 0; o < D; o++) {
    double s = 0.0;
    for (int64_t f = 0; f < F; f++) s += weight(w2, w_fmt, s2, D, F, o, f) * h[f];
    out[o] = s;
  }
}

int oracle_ffn_rows(int64_t n, int64_t D, int64_t F, const void *xr, int x_fmt,
                    const void *w1, const void *w2, int w_fmt,
                    const float *s1, const float *s2, double *out,
                    double *h_out) {
  if (w_fmt == OR_I8 && (!s1 || !s2 || D % OR_GROUP || F % OR_GROUP)) return -1;
#pragma omp parallel
  {
    double *h = (double *)malloc((size_t)(F > 0 ? F : 1) * sizeof(double));
#pragma omp for schedule(dynamic, 1)
    for (int64_t r = 0; r < n; r++) {
      ffn_one_row(D, F, xr, x_fmt, r, w1, w2, w_fmt, s1, s2, h, out + r * D);
      if (h_out) memcpy(h_out + r * F, h, (size_t)F * sizeof(double));
    }
    free(h);
  }
  return 0;
}

/* ------------------------------------------------------------------------
 * Gate-weighted combine.  [DSC] combine(returned, gates) and the equation's
 * sum of p_e E_e(x); [DvS] a dropped assignment contributes nothing and the
 * token reaches the next layer through the residual; [DvS] PR-MoE example
 * (fixed-MLP output plus gate times the expert's residual output).
 *   M[t] = sum over kept j (in rank order) of gates[t,j] * expert_out[t,j]
 *   y[t] = base[t] + M[t]          (base NULL -> 0)
 * expert_out: T x k x D doubles (the expert's output for that assignment;
 * ignored for dropped ones).  m_out (optional) receives M.
 * ---------------------------------------------------------------------- */
int oracle_combine(int64_t T, int64_t D, int64_t k, const int32_t *slots,
                   const double *gates, const double *expert_out,
                   const double *base, double *y, double *m_out) {
  for (int64_t t = 0; t < T; t++)
    for (int64_t o = 0; o < D; o++) {
      double m = 0.0;
      for (int64_t j = 0; j < k; j++)
        if (slots[t * k + j] >= 0)
          m += gates[t * k + j] * expert_out[(t * k + j) * D + o];
      if (m_out) m_out[t * D + o] = m;
      y[t * D + o] = (base ? base[t * D + o] : 0.0) + m;
    }
  return 0;
}

/* ------------------------------------------------------------------------
 * Whole layer, composed from the stages above in the order of [DSC]'s
 * pipeline (router, top-k, capacity dispatch, experts, combine, aux loss).
 *   y = (add_skip ? x : 0) + (pr_moe ? D(x) : 0) + M(x)
 * add_skip: the residual that carries a dropped token on ([DvS] overflow);
 * pr_moe: the fixed dense MLP of Residual-MoE ([DSN] 3.1).
 * Expert weights: w1 [E, F, D], w2 [E, D, F] (int8: scales [E, F, D/128]
 * and [E, D, F/128]); dense MLP wm1 [Fd, D], wm2 [D, Fd] in x_fmt.
 * Outputs (doubles unless noted): logits/probs T x E, ids/slots T x k
 * (int32), gates T x k, drop T x k (uint8), load/kept E (int32),
 * expert_out T x k x D (per assignment; zero when dropped),
 * m T x D, dense T x D (zero when !pr_moe), y T x D, aux [1].
 * ---------------------------------------------------------------------- */
/* the router variants of the section after oracle_z_loss */
int oracle_route_variant(int64_t T, int64_t d, int64_t E, int64_t k, int variant, int normalize,
                         double top_p, double tau, int64_t de, const void *x, int x_fmt,
                         const void *wr, const float *bias, const void *w_noise,
                         const float *noise, const void *emb, double *logits, double *probs,
                         int32_t *ids, double *gates, double *load_p);

/* The layer with a router variant (variant 0 = the softmax router of
 * oracle_route; wr is then W_r, else as oracle_route_variant takes it). */
int oracle_layer_forward_v(int64_t T, int64_t D, int64_t E, int64_t k,
                           int64_t F, int64_t Fd, double cf, int64_t cap_override,
                           int normalize, int pr_moe, int add_skip, int policy,
                           double alpha, const void *x, int x_fmt,
                           const void *wr, const float *bias, const void *w1,
                           const void *w2, int w_fmt, const float *s1,
                           const float *s2, const void *wm1, const void *wm2,
                           double *logits, double *probs, int32_t *ids,
                           double *gates, int32_t *slots, uint8_t *drop,
                           int32_t *load, int32_t *kept, double *expert_out,
                           double *m, double *dense, double *y, double *aux,
                           int variant, double top_p, double tau, int64_t de,
                           const void *w_noise, const float *noise, const void *emb,
                           double *load_p) {
  int rc;
  if (variant == 0)
    rc = oracle_route(T, D, E, k, normalize, x, x_fmt, wr, x_fmt, bias, logits, probs, ids,
                      gates);
  else
    rc = oracle_route_variant(T, D, E, k, variant, normalize, top_p, tau, de, x, x_fmt, wr,
                              bias, w_noise, noise, emb, logits, probs, ids, gates, load_p);
  if (rc) return rc;
  *aux = oracle_aux_loss(T, E, k, ids, probs, alpha, NULL, NULL);
  int64_t C = oracle_capacity(T, E, k, cf, cap_override);
  rc = oracle_dispatch(T, E, k, C, ids, gates, policy, slots, drop, load, kept);
  if (rc) return rc;

  size_t ws = (w_fmt == OR_F64) ? 8 : (w_fmt == OR_F32) ? 4 : (w_fmt == OR_BF16 ? 2 : 1);
  if (w_fmt == OR_I8 && (!s1 || !s2 || D % OR_GROUP || F % OR_GROUP)) return -1;
  memset(expert_out, 0, (size_t)(T * k * D) * sizeof(double));
#pragma omp parallel
  {
    double *h = (double *)malloc((size_t)(F > 0 ? F : 1) * sizeof(double));
#pragma omp for schedule(dynamic, 1)
    for (int64_t a = 0; a < T * k; a++) {
      if (slots[a] < 0) continue;
      int64_t e = ids[a];
      ffn_one_row(D, F, x, x_fmt, a / k,
                  (const char *)w1 + (size_t)(e * F * D) * ws,
                  (const char *)w2 + (size_t)(e * D * F) * ws, w_fmt,
                  s1 ? s1 + e * F * (D / OR_GROUP) : NULL,
                  s2 ? s2 + e * D * (F / OR_GROUP) : NULL, h,
                  expert_out + a * D);
    }
    free(h);
  }

  if (pr_moe) {
    rc = oracle_ffn_rows(T, D, Fd, x, x_fmt, wm1, wm2, x_fmt, NULL, NULL,
                         dense, NULL);
    if (rc) return rc;
  } else {
    memset(dense, 0, (size_t)(T * D) * sizeof(double));
  }
  double *base = (double *)malloc((size_t)(T * D > 0 ? T * D : 1) * sizeof(double));
  for (int64_t t = 0; t < T; t++)
    for (int64_t o = 0; o < D; o++)
      base[t * D + o] = (add_skip ? elem(x, x_fmt, t * D + o) : 0.0) + dense[t * D + o];
  rc = oracle_combine(T, D, k, slots, gates, expert_out, base, y, m);
  free(base);
  return rc;
}

int oracle_layer_forward(int64_t T, int64_t D, int64_t E, int64_t k,
                         int64_t F, int64_t Fd, double cf, int64_t cap_override,
                         int normalize, int pr_moe, int add_skip, int policy,
                         double alpha, const void *x, int x_fmt,
                         const void *wr, const float *bias, const void *w1,
                         const void *w2, int w_fmt, const float *s1,
                         const float *s2, const void *wm1, const void *wm2,
                         double *logits, double *probs, int32_t *ids,
                         double *gates, int32_t *slots, uint8_t *drop,
                         int32_t *load, int32_t *kept, double *expert_out,
                         double *m, double *dense, double *y, double *aux) {
  return oracle_layer_forward_v(T, D, E, k, F, Fd, cf, cap_override, normalize, pr_moe,
                                add_skip, policy, alpha, x, x_fmt, wr, bias, w1, w2, w_fmt, s1,
                                s2, wm1, wm2, logits, probs, ids, gates, slots, drop, load, kept,
                                expert_out, m, dense, y, aux, 0, 0.0, 0.0, 0, NULL, NULL, NULL,
                                NULL);
}

/* ------------------------------------------------------------------------
 * Router z-loss, [DvS] section "Router Z-loss":
 *   L_z = (1/B) sum over tokens of (log sum_j exp(logit_j))^2
 * computed with the max shifted out of the exponentials.
 * ---------------------------------------------------------------------- */
double oracle_z_loss(int64_t T, int64_t E, const double *logits) {
  if (T <= 0) return 0.0;
  double acc = 0.0;
  for (int64_t t = 0; t < T; t++) {
    const double *l = logits + t * E;
    double m = l[0];
    for (int64_t e = 1; e < E; e++)
      if (l[e] > m) m = l[e];
    double s = 0.0;
    for (int64_t e = 0; e < E; e++) s += exp(l[e] - m);
    double lz = m + log(s);
    acc += lz * lz;
  }
  return acc / (double)T;
}

/* ------------------------------------------------------------------------
 * Symmetric int8 quantisation of one [N, K] matrix in groups of 128 along K,
 * [SRV] 1.2.2: s = max|r| / q_max with q_max = 127; q = clamp(round(r / s),
 * -127, 127) with round-half-to-even; a group whose values are all zero gets
 * s = 0 and q = 0.  Scales come out as doubles; a caller that stores them in
 * a narrower format rounds them first and passes that value in scale_in to
 * quantise against it (scale_in NULL: use the exact scale).
 * ---------------------------------------------------------------------- */
int oracle_quantize_sym_int8(int64_t N, int64_t K, const double *w,
                             const double *scale_in, int8_t *q,
                             double *scale_out) {
  if (K % OR_GROUP) return -1;
  int64_t G = K / OR_GROUP;
  for (int64_t n = 0; n < N; n++)
    for (int64_t g = 0; g < G; g++) {
      const double *r = w + n * K + g * OR_GROUP;
      double s;
      if (scale_in) {
        s = scale_in[n * G + g];
      } else {
        double amax = 0.0;
        for (int64_t i = 0; i < OR_GROUP; i++)
          if (fabs(r[i]) > amax) amax = fabs(r[i]);
        s = amax / 127.0;
      }
      if (scale_out) scale_out[n * G + g] = s;
      for (int64_t i = 0; i < OR_GROUP; i++) {
        double v = (s > 0.0) ? nearbyint(r[i] / s) : 0.0; /* default mode: half to even */
        if (v > 127.0) v = 127.0;
        if (v < -127.0) v = -127.0;
        q[n * K + g * OR_GROUP + i] = (int8_t)v;
      }
    }
  return 0;
}

/* ------------------------------------------------------------------------
 * Backward of the layer: the gradients of the scalar
 *   L = sum_{t,o} dy[t,o] y[t,o] + g_aux * aux + g_z * z
 * (z the router z-loss above) with respect to x, W_r, b, W1, W2, Wm1, Wm2,
 * by the chain rule through the forward stages, written out directly.
 *  - A kept assignment (t, j) adds g_tj * E_e(x_t) to y_t, so
 *      dg_tj = <dy_t, E_e(x_t)>   and the expert sees d(out) = g_tj dy_t;
 *    a dropped assignment adds nothing and gets no gradient ([DvS] overflow:
 *    the token skips the expert).
 *  - An FFN out = W2 GELU(W1 x) (the experts, and the PR-MoE dense MLP with
 *    d(out) = dy_t): with a = W1 x and h = GELU(a),
 *      dh = W2^T d(out),  da = dh * GELU'(a),  GELU'(a) = Phi(a) + a phi(a),
 *      dx += W1^T da,  dW2 += d(out) h^T,  dW1 += da x^T.
 *  - Gates from probabilities: g_j = p_{e_j} (k = 1, or no renormalisation);
 *    renormalised ([SRV] 1.1.1.1) g_j = p_{e_j} / S with S the sum of the k
 *    chosen p, so  dp_{e_i} += (dg_i - sum_j dg_j g_j) / S.
 *  - aux = alpha E sum_e f_e Q_e with Q_e = (1/T) sum_t p_e(t) ([SRV]
 *    1.1.4.1); f counts argmax decisions and is piecewise constant:
 *      dp_e(t) += g_aux alpha E f_e / T.
 *  - Softmax: dlogit_e = p_e (dp_e - sum_i p_i dp_i).
 *  - z = (1/T) sum_t lse_t^2: dlogit_e(t) += g_z (2/T) lse_t p_e(t).
 *  - logits = W_r x + b: dx += W_r^T dlogit, dW_r += dlogit x^T, db += dlogit.
 * The discrete decisions (top-k, capacity) are held where the forward put
 * them (their derivative is zero almost everywhere).  Plain weights (x_fmt)
 * only.  Outputs are doubles: dx [T, D], dwr [E, D], db [E] (may be NULL),
 * dw1 [E, F, D], dw2 [E, D, F], dwm1 [Fd, D], dwm2 [D, Fd] (pr_moe only).
 * ---------------------------------------------------------------------- */
static double gelu_grad(double z) {
  const double inv_sqrt_2pi = 0.39894228040143267794;
  return 0.5 * (1.0 + erf(z / sqrt(2.0))) + z * inv_sqrt_2pi * exp(-0.5 * z * z);
}

/* one FFN row backward; accumulates into dx_row, dw1 [F, D], dw2 [D, F] */
static void ffn_row_backward(int64_t D, int64_t F, const void *x, int fmt, int64_t row,
                             const void *w1, const void *w2, const double *dout,
                             double *a, double *dh, double *dx_row, double *dw1,
                             double *dw2) {
  for (int64_t f = 0; f < F; f++) {
    double s = 0.0;
    for (int64_t i = 0; i < D; i++) s += elem(w1, fmt, f * D + i) * elem(x, fmt, row * D + i);
    a[f] = s;
  }
  for (int64_t f = 0; f < F; f++) {
    double s = 0.0;
    for (int64_t o = 0; o < D; o++) s += elem(w2, fmt, o * F + f) * dout[o];
    dh[f] = s * gelu_grad(a[f]); /* da */
  }
  for (int64_t i = 0; i < D; i++) {
    double s = 0.0;
    for (int64_t f = 0; f < F; f++) s += elem(w1, fmt, f * D + i) * dh[f];
    dx_row[i] += s;
  }
  if (!dw1 || !dw2) return; /* dx only */
  for (int64_t f = 0; f < F; f++) {
    const double hf = gelu(a[f]);
    for (int64_t o = 0; o < D; o++) dw2[o * F + f] += dout[o] * hf;
  }
  for (int64_t f = 0; f < F; f++)
    for (int64_t i = 0; i < D; i++) dw1[f * D + i] += dh[f] * elem(x, fmt, row * D + i);
}

/* dL/dlogits of one token from its gate gradients dg_j = <dy_t, expert output>
 * (zero for a dropped assignment), its chosen experts ids_t, gates g, softmax
 * probabilities p, log-sum-exp lse and the argmax fractions f; dp is scratch
 * [E], the result goes to dl [E] (the bullets above, in order). */
static void router_token_grad(int64_t E, int64_t k, int64_t T, int normalize, double alpha,
                              double g_aux, double g_z, const double *f, const double *p,
                              double lse, const int32_t *ids_t, const double *g,
                              const double *dg, double *dp, double *dl) {
  for (int64_t e = 0; e < E; e++) dp[e] = g_aux * alpha * (double)E * f[e] / (double)T;
  double S = 0.0, sdg = 0.0;
  for (int64_t j = 0; j < k; j++) {
    S += p[ids_t[j]];
    sdg += dg[j] * g[j];
  }
  for (int64_t j = 0; j < k; j++)
    dp[ids_t[j]] += (k >= 2 && normalize) ? (dg[j] - sdg) / S : dg[j];
  double pdp = 0.0;
  for (int64_t e = 0; e < E; e++) pdp += p[e] * dp[e];
  for (int64_t e = 0; e < E; e++)
    dl[e] = p[e] * (dp[e] - pdp) + g_z * 2.0 / (double)T * lse * p[e];
}

int oracle_layer_backward(int64_t T, int64_t D, int64_t E, int64_t k, int64_t F,
                          int64_t Fd, double cf, int64_t cap_override, int normalize,
                          int pr_moe, int add_skip, int policy, double alpha,
                          const void *x, int fmt, const void *wr, const float *bias,
                          const void *w1, const void *w2, const void *wm1, const void *wm2,
                          const double *dy, double g_aux, double g_z, double *dx,
                          double *dwr, double *db, double *dw1, double *dw2,
                          double *dwm1, double *dwm2) {
  if (fmt == OR_I8) return -1;
  const int64_t TE = T * E > 0 ? T * E : 1, Tk = T * k > 0 ? T * k : 1;
  const int64_t TD = T * D > 0 ? T * D : 1;
  double *logits = (double *)malloc((size_t)TE * sizeof(double));
  double *probs = (double *)malloc((size_t)TE * sizeof(double));
  int32_t *ids = (int32_t *)malloc((size_t)Tk * sizeof(int32_t));
  double *gates = (double *)malloc((size_t)Tk * sizeof(double));
  int32_t *slots = (int32_t *)malloc((size_t)Tk * sizeof(int32_t));
  uint8_t *drop = (uint8_t *)malloc((size_t)Tk);
  int32_t *load = (int32_t *)malloc((size_t)(E > 0 ? E : 1) * sizeof(int32_t));
  int32_t *kept = (int32_t *)malloc((size_t)(E > 0 ? E : 1) * sizeof(int32_t));
  double *eo = (double *)malloc((size_t)(Tk * D) * sizeof(double));
  double *m = (double *)malloc((size_t)TD * sizeof(double));
  double *dense = (double *)malloc((size_t)TD * sizeof(double));
  double *y = (double *)malloc((size_t)TD * sizeof(double));
  double *f = (double *)calloc((size_t)(E > 0 ? E : 1), sizeof(double));
  double *dxa = (double *)calloc((size_t)(Tk * D), sizeof(double)); /* per assignment */
  double *dlog = (double *)calloc((size_t)TE, sizeof(double));
  double aux = 0.0;
  int rc = oracle_layer_forward(T, D, E, k, F, Fd, cf, cap_override, normalize, pr_moe,
                                add_skip, policy, alpha, x, fmt, wr, bias, w1, w2, fmt, NULL,
                                NULL, wm1, wm2, logits, probs, ids, gates, slots, drop, load,
                                kept, eo, m, dense, y, &aux);
  if (rc) goto done;
  oracle_aux_loss(T, E, k, ids, probs, alpha, f, NULL);
  const size_t es = fmt == OR_F64 ? 8 : (fmt == OR_F32 ? 4 : 2);

  /* experts: each expert's kept assignments in token order */
  memset(dw1, 0, (size_t)(E * F * D) * sizeof(double));
  memset(dw2, 0, (size_t)(E * D * F) * sizeof(double));
#pragma omp parallel
  {
    double *a = (double *)malloc((size_t)(F > 0 ? F : 1) * sizeof(double));
    double *dh = (double *)malloc((size_t)(F > 0 ? F : 1) * sizeof(double));
    double *dout = (double *)malloc((size_t)(D > 0 ? D : 1) * sizeof(double));
#pragma omp for schedule(dynamic, 1)
    for (int64_t e = 0; e < E; e++) {
      const void *w1e = (const char *)w1 + (size_t)(e * F * D) * es;
      const void *w2e = (const char *)w2 + (size_t)(e * D * F) * es;
      for (int64_t q = 0; q < T * k; q++) {
        if (ids[q] != e || slots[q] < 0) continue;
        const int64_t t = q / k;
        for (int64_t o = 0; o < D; o++) dout[o] = gates[q] * dy[t * D + o];
        ffn_row_backward(D, F, x, fmt, t, w1e, w2e, dout, a, dh, dxa + q * D,
                         dw1 + e * F * D, dw2 + e * D * F);
      }
    }
    free(a);
    free(dh);
    free(dout);
  }

  /* dense MLP over every token */
  if (pr_moe) {
    memset(dwm1, 0, (size_t)(Fd * D) * sizeof(double));
    memset(dwm2, 0, (size_t)(D * Fd) * sizeof(double));
    double *a = (double *)malloc((size_t)(Fd > 0 ? Fd : 1) * sizeof(double));
    double *dh = (double *)malloc((size_t)(Fd > 0 ? Fd : 1) * sizeof(double));
    memset(dx, 0, (size_t)TD * sizeof(double));
    for (int64_t t = 0; t < T; t++)
      ffn_row_backward(D, Fd, x, fmt, t, wm1, wm2, dy + t * D, a, dh, dx + t * D, dwm1, dwm2);
    free(a);
    free(dh);
  } else {
    memset(dx, 0, (size_t)TD * sizeof(double));
  }

  /* router: gates -> probabilities -> logits */
#pragma omp parallel
  {
    double *dp = (double *)malloc((size_t)(E > 0 ? E : 1) * sizeof(double));
#pragma omp for schedule(static)
    for (int64_t t = 0; t < T; t++) {
      const double *p = probs + t * E, *l = logits + t * E;
      double dg[64];
      for (int64_t j = 0; j < k; j++) {
        const int64_t q = t * k + j;
        double v = 0.0;
        if (slots[q] >= 0)
          for (int64_t o = 0; o < D; o++) v += dy[t * D + o] * eo[q * D + o];
        dg[j] = v;
      }
      double mx = l[0];
      for (int64_t e = 1; e < E; e++)
        if (l[e] > mx) mx = l[e];
      double se = 0.0;
      for (int64_t e = 0; e < E; e++) se += exp(l[e] - mx);
      router_token_grad(E, k, T, normalize, alpha, g_aux, g_z, f, p, mx + log(se), ids + t * k,
                        gates + t * k, dg, dp, dlog + t * E);
    }
    free(dp);
  }
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; t++)
    for (int64_t i = 0; i < D; i++) {
      double s = add_skip ? dy[t * D + i] : 0.0;
      for (int64_t j = 0; j < k; j++) s += dxa[(t * k + j) * D + i];
      for (int64_t e = 0; e < E; e++) s += dlog[t * E + e] * elem(wr, fmt, e * D + i);
      dx[t * D + i] += s;
    }
#pragma omp parallel for schedule(static)
  for (int64_t e = 0; e < E; e++) {
    for (int64_t i = 0; i < D; i++) {
      double s = 0.0;
      for (int64_t t = 0; t < T; t++) s += dlog[t * E + e] * elem(x, fmt, t * D + i);
      dwr[e * D + i] = s;
    }
    if (db) {
      double s = 0.0;
      for (int64_t t = 0; t < T; t++) s += dlog[t * E + e];
      db[e] = s;
    }
  }
done:
  free(logits); free(probs); free(ids); free(gates); free(slots); free(drop); free(load);
  free(kept); free(eo); free(m); free(dense); free(y); free(f); free(dxa); free(dlog);
  return rc;
}

/* ------------------------------------------------------------------------
 * Selected entries of the layer backward, for checks at sizes where the
 * whole backward is too slow: the chain rule of oracle_layer_backward
 * restricted to
 *   the dx rows of the tokens in `rows`, and
 *   dW1[e][f][i] and dW2[e][o][f] entries listed as (e, ., .) triples,
 * given the forward's discrete decisions ids and slots (for example another
 * implementation's), with every continuous value (logits, probabilities,
 * gates, expert activations and outputs) recomputed in fp64 from x and the
 * weights; f (argmax fractions of the aux loss) from ids[t, 0].
 * Plain weights only.  dy: T x D (every token's, the dW sums read them
 * all); dx_rows: n_rows x D; dw1_vals, dw2_vals: one per triple.
 * ---------------------------------------------------------------------- */
/* probabilities, log-sum-exp and gates of token t under the given ids */
static void token_gates(int64_t D, int64_t E, int64_t k, int normalize, const void *x, int fmt,
                        const void *wr, const float *bias, const int32_t *ids, int64_t t,
                        double *p, double *lse, double *g) {
  double mx = -INFINITY;
  for (int64_t e = 0; e < E; e++) {
    double s = 0.0;
    for (int64_t i = 0; i < D; i++) s += elem(x, fmt, t * D + i) * elem(wr, fmt, e * D + i);
    if (bias) s += (double)bias[e];
    p[e] = s;
    if (s > mx) mx = s;
  }
  double z = 0.0;
  for (int64_t e = 0; e < E; e++) z += exp(p[e] - mx);
  *lse = mx + log(z);
  for (int64_t e = 0; e < E; e++) p[e] = exp(p[e] - *lse);
  double S = 0.0;
  for (int64_t j = 0; j < k; j++) S += p[ids[t * k + j]];
  for (int64_t j = 0; j < k; j++)
    g[j] = (k >= 2 && normalize) ? p[ids[t * k + j]] / S : p[ids[t * k + j]];
}

int oracle_backward_sampled(int64_t T, int64_t D, int64_t E, int64_t k, int64_t F, int64_t Fd,
                            int normalize, int pr_moe, int add_skip, double alpha,
                            const void *x, int fmt, const void *wr, const float *bias,
                            const void *w1, const void *w2, const void *wm1, const void *wm2,
                            const int32_t *ids, const int32_t *slots, const double *dy,
                            double g_aux, double g_z, const int64_t *rows, int64_t n_rows,
                            double *dx_rows, const int64_t *w1_idx, int64_t n_w1,
                            double *dw1_vals, const int64_t *w2_idx, int64_t n_w2,
                            double *dw2_vals) {
  if (fmt == OR_I8 || k > 64) return -1;
  const size_t es = fmt == OR_F64 ? 8 : (fmt == OR_F32 ? 4 : 2);
  double *f = (double *)calloc((size_t)(E > 0 ? E : 1), sizeof(double));
  for (int64_t t = 0; t < T; t++) f[ids[t * k]] += 1.0 / (double)T;
  const int64_t Fm = F > Fd ? F : Fd;
  int rc = 0;

  /* dx rows */
#pragma omp parallel
  {
    double *p = (double *)malloc((size_t)E * sizeof(double));
    double *dp = (double *)malloc((size_t)E * sizeof(double));
    double *dl = (double *)malloc((size_t)E * sizeof(double));
    double *a = (double *)malloc((size_t)(Fm > 0 ? Fm : 1) * sizeof(double));
    double *dh = (double *)malloc((size_t)(Fm > 0 ? Fm : 1) * sizeof(double));
    double *o = (double *)malloc((size_t)D * sizeof(double));
    double *dout = (double *)malloc((size_t)D * sizeof(double));
#pragma omp for schedule(dynamic, 1)
    for (int64_t n = 0; n < n_rows; n++) {
      const int64_t t = rows[n];
      double *dx = dx_rows + n * D;
      const double *dyt = dy + t * D;
      double lse, g[64], dg[64];
      token_gates(D, E, k, normalize, x, fmt, wr, bias, ids, t, p, &lse, g);
      for (int64_t i = 0; i < D; i++) dx[i] = add_skip ? dyt[i] : 0.0;
      if (pr_moe) ffn_row_backward(D, Fd, x, fmt, t, wm1, wm2, dyt, a, dh, dx, NULL, NULL);
      for (int64_t j = 0; j < k; j++) {
        const int64_t q = t * k + j, e = ids[q];
        dg[j] = 0.0;
        if (slots[q] < 0) continue;
        const void *w1e = (const char *)w1 + (size_t)(e * F * D) * es;
        const void *w2e = (const char *)w2 + (size_t)(e * D * F) * es;
        ffn_one_row(D, F, x, fmt, t, w1e, w2e, fmt, NULL, NULL, a, o);
        for (int64_t i = 0; i < D; i++) dg[j] += dyt[i] * o[i];
        for (int64_t i = 0; i < D; i++) dout[i] = g[j] * dyt[i];
        ffn_row_backward(D, F, x, fmt, t, w1e, w2e, dout, a, dh, dx, NULL, NULL);
      }
      router_token_grad(E, k, T, normalize, alpha, g_aux, g_z, f, p, lse, ids + t * k, g, dg, dp,
                        dl);
      for (int64_t e = 0; e < E; e++)
        for (int64_t i = 0; i < D; i++) dx[i] += dl[e] * elem(wr, fmt, e * D + i);
    }
    free(p); free(dp); free(dl); free(a); free(dh); free(o); free(dout);
  }

  /* expert weight-gradient entries: sums over the expert's kept assignments */
#pragma omp parallel
  {
    double *p = (double *)malloc((size_t)E * sizeof(double));
#pragma omp for schedule(dynamic, 1)
    for (int64_t n = 0; n < n_w1 + n_w2; n++) {
      const int is1 = n < n_w1;
      const int64_t *ix = is1 ? w1_idx + 3 * n : w2_idx + 3 * (n - n_w1);
      const int64_t e = ix[0];
      const int64_t fi = is1 ? ix[1] : ix[2]; /* hidden unit */
      const void *w1e = (const char *)w1 + (size_t)(e * F * D) * es;
      const void *w2e = (const char *)w2 + (size_t)(e * D * F) * es;
      double acc = 0.0, lse, g[64];
      for (int64_t q = 0; q < T * k; q++) {
        if (slots[q] < 0 || ids[q] != e) continue; /* kept rows of e */
        const int64_t t = q / k, j = q % k;
        token_gates(D, E, k, normalize, x, fmt, wr, bias, ids, t, p, &lse, g);
        double av = 0.0;
        for (int64_t i = 0; i < D; i++) av += elem(w1e, fmt, fi * D + i) * elem(x, fmt, t * D + i);
        if (is1) { /* dW1[e][f][i] = sum da_f x_i, da_f = GELU'(a_f) sum_o W2[o][f] g dy[o] */
          double s = 0.0;
          for (int64_t o2 = 0; o2 < D; o2++) s += elem(w2e, fmt, o2 * F + fi) * g[j] * dy[t * D + o2];
          acc += s * gelu_grad(av) * elem(x, fmt, t * D + ix[2]);
        } else { /* dW2[e][o][f] = sum g dy[o] GELU(a_f) */
          acc += g[j] * dy[t * D + ix[1]] * gelu(av);
        }
      }
      if (is1) dw1_vals[n] = acc;
      else dw2_vals[n - n_w1] = acc;
    }
    free(p);
  }
  free(f);
  return rc;
}

/* ------------------------------------------------------------------------
 * Router variants ([SRV2]), each followed by the same capacity dispatch,
 * experts and combine as the softmax router.  variant:
 *   OR_ROUTER_TOPK   logits = W_r x (+ b); TopK as oracle_route.
 *   OR_ROUTER_TOP_P  logits = W_r x (+ b), p = softmax; experts are taken in
 *                    descending p (ties to the lower index), accumulating
 *                    their p, until the sum exceeds top_p ("until the
 *                    cumulative value exceeds P, activate every accumulated
 *                    expert", sec. 1.1.4.2); at most k are taken (the k slots
 *                    per token); unused slots get id -1 and gate 0.  Gates:
 *                    normalize -> p over the sum of the taken p (any count),
 *                    else p.
 *   OR_ROUTER_COSINE u = W_proj x (de values); logit_e = <emb_e, u> /
 *                    (tau |u| |emb_e|) (+ b), 0 when a norm is 0 (sec.
 *                    1.1.1.2: the token's projection against each expert's
 *                    embedding, sharpened by 1/tau); softmax and TopK as the
 *                    softmax router.
 *   OR_ROUTER_NOISY  clean_e = W_g x (+ b), sigma_e = softplus(W_noise x),
 *                    H_e = clean_e + eps_e sigma_e with eps the caller's
 *                    standard-normal draws (sec. 1.1.1.1: g linear plus a
 *                    noise term); the k largest H are kept and the gates are
 *                    the softmax over the kept H (TopK before softmax); the
 *                    logits reported are H.
 * load_p[t,e] = P(x_t, e) of the Load loss (sec. 1.1.4.1: the probability
 * that the gate of e is nonzero under a new draw of the noise): for the
 * noisy router, with the other experts' H held, e is kept iff
 * clean_e + eps' sigma_e exceeds the k-th largest H among the other
 * experts, so P = Phi((clean_e - that value) / sigma_e) (1 when fewer than
 * k other experts exist); for the noise-free routers P is 1 if e was taken
 * and 0 otherwise.
 * Formats: x, wr (W_r, W_g or W_proj [de, d]), w_noise [E, d] and emb
 * [E, de] in x_fmt; noise [T, E] float32.
 * ---------------------------------------------------------------------- */
enum { OR_ROUTER_TOPK = 0, OR_ROUTER_TOP_P = 1, OR_ROUTER_COSINE = 2, OR_ROUTER_NOISY = 3 };

static double softplus(double z) { return z > 0.0 ? z + log1p(exp(-z)) : log1p(exp(z)); }
static double std_normal_cdf(double z) { return 0.5 * erfc(-z / sqrt(2.0)); }

int oracle_route_variant(int64_t T, int64_t d, int64_t E, int64_t k, int variant, int normalize,
                         double top_p, double tau, int64_t de, const void *x, int x_fmt,
                         const void *wr, const float *bias, const void *w_noise,
                         const float *noise, const void *emb, double *logits, double *probs,
                         int32_t *ids, double *gates, double *load_p) {
  if (k < 1 || k > E || k > 64) return -1;
  if (variant == OR_ROUTER_TOP_P && !(top_p > 0.0)) return -1;
  if (variant == OR_ROUTER_COSINE && (!(tau > 0.0) || de < 1 || !emb)) return -1;
  if (variant == OR_ROUTER_NOISY && (!w_noise || !noise)) return -1;
  if (variant < OR_ROUTER_TOPK || variant > OR_ROUTER_NOISY) return -1;
  int rc = 0;
#pragma omp parallel
  {
    double *clean = (double *)malloc((size_t)E * sizeof(double));
    double *sigma = (double *)malloc((size_t)E * sizeof(double));
    double *u = (double *)malloc((size_t)(de > 0 ? de : 1) * sizeof(double));
    double *other = (double *)malloc((size_t)E * sizeof(double));
#pragma omp for schedule(dynamic, 4)
    for (int64_t t = 0; t < T; t++) {
      double *l = logits + t * E, *p = probs + t * E;
      /* logits */
      if (variant == OR_ROUTER_COSINE) {
        double nu = 0.0;
        for (int64_t j = 0; j < de; j++) {
          double v = 0.0;
          for (int64_t i = 0; i < d; i++) v += elem(wr, x_fmt, j * d + i) * elem(x, x_fmt, t * d + i);
          u[j] = v;
          nu += v * v;
        }
        nu = sqrt(nu);
        for (int64_t e = 0; e < E; e++) {
          double ne = 0.0, dot = 0.0;
          for (int64_t j = 0; j < de; j++) {
            const double v = elem(emb, x_fmt, e * de + j);
            ne += v * v;
            dot += v * u[j];
          }
          ne = sqrt(ne);
          l[e] = (nu > 0.0 && ne > 0.0) ? dot / (tau * nu * ne) : 0.0;
          if (bias) l[e] += (double)bias[e];
        }
      } else {
        for (int64_t e = 0; e < E; e++) {
          double v = 0.0;
          for (int64_t i = 0; i < d; i++) v += elem(x, x_fmt, t * d + i) * elem(wr, x_fmt, e * d + i);
          if (bias) v += (double)bias[e];
          clean[e] = v;
          l[e] = v;
        }
        if (variant == OR_ROUTER_NOISY)
          for (int64_t e = 0; e < E; e++) {
            double z = 0.0;
            for (int64_t i = 0; i < d; i++)
              z += elem(x, x_fmt, t * d + i) * elem(w_noise, x_fmt, e * d + i);
            sigma[e] = softplus(z);
            l[e] = clean[e] + (double)noise[t * E + e] * sigma[e];
          }
      }
      /* softmax, the largest logit shifted out */
      double lmax = l[0];
      for (int64_t e = 1; e < E; e++)
        if (l[e] > lmax) lmax = l[e];
      double zsum = 0.0;
      for (int64_t e = 0; e < E; e++) zsum += exp(l[e] - lmax);
      for (int64_t e = 0; e < E; e++) p[e] = exp(l[e] - lmax) / zsum;
      /* selection in the order (larger logit, then smaller index) */
      int32_t *sel = ids + t * k;
      int64_t n = 0;
      double cum = 0.0;
      for (int64_t j = 0; j < k; j++) {
        int64_t best = -1;
        for (int64_t e = 0; e < E; e++) {
          int taken = 0;
          for (int64_t q = 0; q < j; q++)
            if (sel[q] == e) taken = 1;
          if (!taken && (best < 0 || l[e] > l[best])) best = e;
        }
        sel[j] = (int32_t)best;
        n = j + 1;
        cum += p[best];
        if (variant == OR_ROUTER_TOP_P && cum > top_p) break;
      }
      for (int64_t j = n; j < k; j++) sel[j] = -1;
      double den = 0.0;
      for (int64_t j = 0; j < n; j++) den += p[sel[j]];
      double *g = gates + t * k;
      for (int64_t j = 0; j < k; j++) {
        if (j >= n) {
          g[j] = 0.0;
          continue;
        }
        int renorm;
        if (variant == OR_ROUTER_NOISY) renorm = 1;
        else if (variant == OR_ROUTER_TOP_P) renorm = normalize;
        else renorm = k >= 2 && normalize;
        g[j] = renorm ? p[sel[j]] / den : p[sel[j]];
      }
      /* P(x, e) */
      if (load_p) {
        double *lp = load_p + t * E;
        for (int64_t e = 0; e < E; e++) {
          int chosen = 0;
          for (int64_t j = 0; j < n; j++)
            if (sel[j] == e) chosen = 1;
          if (variant != OR_ROUTER_NOISY) {
            lp[e] = chosen ? 1.0 : 0.0;
            continue;
          }
          /* k-th largest H among the other experts */
          int64_t no = 0;
          for (int64_t j = 0; j < E; j++)
            if (j != e) other[no++] = l[j];
          if (no < k) {
            lp[e] = 1.0;
            continue;
          }
          for (int64_t a = 0; a < k; a++) /* partial selection sort, descending */
            for (int64_t b = a + 1; b < no; b++)
              if (other[b] > other[a]) {
                const double tmp = other[a];
                other[a] = other[b];
                other[b] = tmp;
              }
          lp[e] = std_normal_cdf((clean[e] - other[k - 1]) / sigma[e]);
        }
      }
    }
    free(clean); free(sigma); free(u); free(other);
  }
  return rc;
}

/* Importance_e = sum over tokens of the gate of e (0 when not chosen), and
 * Load_e = sum over tokens of P(x, e) ([SRV2] 1.1.4.1). */
void oracle_importance_load(int64_t T, int64_t E, int64_t k, const int32_t *ids,
                            const double *gates, const double *load_p, double *importance,
                            double *load) {
  for (int64_t e = 0; e < E; e++) {
    importance[e] = 0.0;
    load[e] = 0.0;
  }
  for (int64_t t = 0; t < T; t++) {
    for (int64_t j = 0; j < k; j++) {
      const int32_t e = ids[t * k + j];
      if (e >= 0 && e < E) importance[e] += gates[t * k + j];
    }
    for (int64_t e = 0; e < E; e++) load[e] += load_p[t * E + e];
  }
}

/* CoV^2 = variance / mean^2 over the n values (population variance: the
 * coefficient of variation of the experts' own values, sec. 1.1.4.1); 0 when
 * the mean is 0. */
double oracle_cov2(int64_t n, const double *v) {
  if (n <= 0) return 0.0;
  double mean = 0.0;
  for (int64_t i = 0; i < n; i++) mean += v[i];
  mean /= (double)n;
  if (mean == 0.0) return 0.0;
  double var = 0.0;
  for (int64_t i = 0; i < n; i++) var += (v[i] - mean) * (v[i] - mean);
  var /= (double)n;
  return var / (mean * mean);
}

/* Number of threads the OpenMP loops above run on (reported with timings of
 * the oracle; not part of the layer's arithmetic). */
int oracle_threads(void) {
  int n = 1;
#ifdef _OPENMP
#pragma omp parallel
  {
#pragma omp single
    n = omp_get_num_threads();
  }
#endif
  return n;
}
