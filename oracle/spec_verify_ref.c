/*
 * spec_verify_ref.c -- plain fp64 CPU oracle for batched speculative-sampling
 * verification (chain drafts, one correction-or-bonus draw per sequence).
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the checker, not the product: only
 * the test suite, the smoke check and the benchmark's CPU-baseline leg may
 * load the library built from it.  It shares no code, header, table or
 * constant with the HIP library, and the HIP library never calls it.
 *
 * It is written to be read against the pages, not to be fast: every row is
 * turned into a double array, every probability is a double, every sum runs
 * in increasing vocabulary order, and a sort of a copy of the row gives the
 * top-k threshold.  Parallelism (OpenMP) is over independent sequences only.
 *
 * Sources, cited by page title and section:
 *   [WY] "Speculative Decoding 的朴素思想" (whoami-wesleyyou.top, 3.speculativedecoding)
 *        sections "从 LM head 到 sampling distribution", "一次 sampling 怎么执行",
 *        "为什么接受概率恰好是这个比值", "Correction 为什么用正残差",
 *        "从单个 token 接到一段 draft".
 *   [WC] "推测解码：接受规则、状态与收益边界" (wineandchord.com)
 *        sections "两模型精确采样", "单位置接受 reference", "与 Logit Processor 的组合",
 *        "正确性契约".
 *   [TL] tannlonggtaoo.github.io speculative-decoding note, sections
 *        "验证方式：reject sampling", "算法", "Greedy Sampling".
 *
 * Readings where the pages are silent or disagree (each one is listed with its
 * reason in the design notes of the repository):
 *   R1 acceptance: accept iff p(x) > 0 and U <= min(1, p(x)/q(x))   ([WY] step 4 uses <=;
 *      [WC]'s single-position reference needs U = 0 with p(x) = 0 to reject).
 *   R2 uniforms must lie in [0, 1)                                   ([WC] reference).
 *   R3 inverse CDF over half-open cumulative intervals in index order
 *      ([WY] step 1: a uniform picks the token whose cumulative interval holds it).
 *   R4 a rejection whose residual mass is exactly zero draws the correction from p_j
 *      itself ([WC] "正确性契约" asks for a stable fallback without fixing one).  Valid
 *      inputs reach it when p and q differ only at tokens whose mass is lost against the
 *      partition in double precision (a logit of -460 drafted with -459): then p <= q
 *      everywhere after rounding, and p restricted to the other tokens is the exact law.
 *   R5 top-k keeps every logit >= the k-th largest raw logit (ties kept), applied to
 *      target and draft alike, before temperature; k <= 0 or k >= V disables it.
 *   R6 temperature 0 is greedy: argmax with the lowest index on ties; draft logits and
 *      uniforms are not read ([WY] LM-head section; [TL] "Greedy Sampling").
 *   R7 "p(x) > 0" / "q(x) = 0" are support tests (kept by top-k and a finite logit);
 *      the ratio itself is formed as exp(min(0, log p(x) - log q(x))), which is
 *      min(1, p/q) written so that neither side underflows.
 *   R16 tree verification: node 0 is the root (the committed context) and every other node n
 *      has a parent parent[n] < n and a token x_n; p_u (target row u) is the target's
 *      distribution after node u's path and q_u (draft row u) the distribution u's
 *      children were drawn from, independently and with replacement.  The walk starts at
 *      the root and tests u's children in index order against the current distribution
 *      (p_u at first); each rejection replaces it by norm([cur - q_u]_+) before the next
 *      sibling (SpecInfer's multi-step sampling as "Speculative Decoding 的朴素思想",
 *      "Token Tree Verifier", describes it; EAGLE's recursive rejection on the EAGLE page,
 *      section 6.2).  An accepted child becomes the new u; when every child is rejected
 *      the token is drawn from the current distribution; at a leaf the bonus comes from
 *      p_u.  Greedy (T = 0): the first child whose token is argmax p_u is accepted, else
 *      argmax p_u is emitted.
 *   R17 typical acceptance ("Speculative Decoding 的朴素思想", section "Medusa-1 与 typical
 *      acceptance"): drafted token x_i is accepted when p_i(x_i) > min(eps, delta *
 *      exp(-H(p_i))), H the entropy (natural log) of the policy distribution p_i; the
 *      accepted prefix is the longest run of accepted positions, and the token after it
 *      is the target's greedy choice argmax p_{j+1} (the "first token, greedy, accepted
 *      directly" of the next candidate).  Defined for T > 0; eps, delta >= 0 are the
 *      caller's.  Not distribution-preserving (the same section says so).
 *   R15 the overlap of a position is taken between the two distributions the
 *      verification compares there: p_i and q_i after the same temperature and top-k.
 *      It is defined for T > 0 only (at T = 0 the policy is a deterministic choice).
 *      TV is summed from its own definition, not as 1 - beta.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define REF_F32 0
#define REF_BF16 1

/* row error codes written into accepted_len[b] (same meaning as the library's) */
#define REF_ERR_TOKEN (-1)    /* drafted token outside [0, V)                      */
#define REF_ERR_QZERO (-2)    /* drafted token has q(x) = 0: the draft cannot emit it */
#define REF_ERR_ROW (-3)      /* NaN or +inf logit, or a row with no finite logit   */
#define REF_ERR_UNIFORM (-4)  /* a uniform outside [0, 1)                            */
#define REF_ERR_TREE (-6)     /* parent array not a tree in topological order       */

/* ---- reading stored logits ------------------------------------------------ */

/* A bf16 value is the upper 16 bits of an IEEE binary32; both convert to double exactly. */
static double logit_at(const void *base, int dtype, size_t idx) {
  if (dtype == REF_F32) return (double)((const float *)base)[idx];
  uint32_t bits = (uint32_t)((const uint16_t *)base)[idx] << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

static void load_row(const void *base, int dtype, size_t row, int V, double *z) {
  for (int v = 0; v < V; ++v) z[v] = logit_at(base, dtype, row * (size_t)V + (size_t)v);
}

/* A row is usable when no logit is NaN or +inf and at least one logit is finite. */
static int row_is_valid(const double *z, int V) {
  int any_finite = 0;
  for (int v = 0; v < V; ++v) {
    if (isnan(z[v]) || z[v] == INFINITY) return 0;
    if (isfinite(z[v])) any_finite = 1;
  }
  return any_finite;
}

/* ---- sampling policy: logits -> distribution ([WY] LM-head section; [WC] logit processors) */

static int cmp_desc(const void *a, const void *b) {
  double x = *(const double *)a, y = *(const double *)b;
  return (x < y) - (x > y);
}

/* k-th largest value of z counting multiplicity (R5): sort a copy, descending. */
double ref_topk_threshold_d(const double *z, int V, int k) {
  double *tmp = (double *)malloc(sizeof(double) * (size_t)V);
  memcpy(tmp, z, sizeof(double) * (size_t)V);
  qsort(tmp, (size_t)V, sizeof(double), cmp_desc);
  double tau = tmp[k - 1];
  free(tmp);
  return tau;
}

static int topk_active(int V, int k) { return k > 0 && k < V; }

/* Policy of one row for temperature T > 0 (R5): keep[v] = 1 for kept v;
 * returns the log-partition L = m + ln S of the kept scaled logits z/T, and
 * writes P[v] = exp(z_v/T - m) / S (0 outside the kept set).  S is summed in
 * increasing v.  keep / P may be NULL. */
static double policy(const double *z, int V, double T, int k, unsigned char *keep, double *P) {
  double tau = topk_active(V, k) ? ref_topk_threshold_d(z, V, k) : -INFINITY;
  double m = -INFINITY;
  for (int v = 0; v < V; ++v) {
    int kept = (z[v] >= tau) && (z[v] > -INFINITY);
    if (keep) keep[v] = (unsigned char)kept;
    if (kept && z[v] / T > m) m = z[v] / T;
  }
  double S = 0.0;
  for (int v = 0; v < V; ++v) {
    int kept = (z[v] >= tau) && (z[v] > -INFINITY);
    double e = kept ? exp(z[v] / T - m) : 0.0;
    if (P) P[v] = e;
    S += e;
  }
  if (P)
    for (int v = 0; v < V; ++v) P[v] /= S;
  return m + log(S);
}

/* Greedy policy (R6): all mass on the argmax, lowest index on ties. */
static int argmax_lowest(const double *z, int V) {
  int a = 0;
  for (int v = 1; v < V; ++v)
    if (z[v] > z[a]) a = v;
  return a;
}

/* ---- inverse CDF ([WY] "一次 sampling 怎么执行" step 1; R3) -------------------- */

/* Returns min{v : F_v > u * F_{V-1}} where F is the running sum of w in increasing v.
 * If rounding leaves no such v, returns the largest v with w_v > 0.  *dist receives
 * the distance of t = u*total to the nearer edge of the chosen interval, divided by
 * the total (the "boundary distance" used to classify parity mismatches).  Returns -1
 * when the total mass is zero. */
int ref_invcdf(const double *w, int V, double u, double *dist) {
  double total = 0.0;
  for (int v = 0; v < V; ++v) total += w[v];
  if (!(total > 0.0)) {
    if (dist) *dist = 0.0;
    return -1;
  }
  double t = u * total;
  double F = 0.0, Fprev = 0.0;
  for (int v = 0; v < V; ++v) {
    Fprev = F;
    F += w[v];
    if (F > t) {
      if (dist) *dist = fmin(t - Fprev, F - t) / total;
      return v;
    }
  }
  int last = V - 1;
  while (last > 0 && !(w[last] > 0.0)) --last;
  if (dist) *dist = 0.0;
  return last;
}

/* ---- one sequence ---------------------------------------------------------- */

typedef struct {
  const void *target, *draft;
  int dtype;
  const int32_t *tokens;
  const float *u_accept, *u_sample;
  int B, G, V;
  double T;
  int k;
  int32_t *accepted_len, *out_tokens;
  double *row_logz, *accept_margin, *sample_margin;
} job_t;

static void fill_tokens(int32_t *out, int n, int32_t value) {
  for (int i = 0; i < n; ++i) out[i] = value;
}

static void verify_sequence(const job_t *J, int b, double *zt, double *zd, double *P, double *Q,
                            double *W, unsigned char *keep_t, unsigned char *keep_d) {
  const int G = J->G, V = J->V;
  const int greedy = (J->T == 0.0);
  int32_t *out = J->out_tokens + (size_t)b * (size_t)(G + 1);
  const int32_t *x = J->tokens + (size_t)b * (size_t)G;
  const size_t trow0 = (size_t)b * (size_t)(G + 1), drow0 = (size_t)b * (size_t)G;

  if (J->accept_margin)
    for (int i = 0; i < G; ++i) J->accept_margin[(size_t)b * G + i] = NAN;
  if (J->sample_margin) J->sample_margin[b] = NAN;

  /* Optional normalisers of every row, for comparing the library's row statistics. */
  if (J->row_logz && !greedy) {
    double *L = J->row_logz + (size_t)b * (size_t)(2 * G + 1);
    for (int i = 0; i <= G; ++i) {
      load_row(J->target, J->dtype, trow0 + i, V, zt);
      L[i] = row_is_valid(zt, V) ? policy(zt, V, J->T, J->k, NULL, NULL) : NAN;
    }
    for (int i = 0; i < G; ++i) {
      load_row(J->draft, J->dtype, drow0 + i, V, zd);
      L[G + 1 + i] = row_is_valid(zd, V) ? policy(zd, V, J->T, J->k, NULL, NULL) : NAN;
    }
  }

  /* Validation, in the order of [WC]'s single-position reference: token range, then
   * the distributions, then the uniform, then "the draft could have sampled x". */
  int err = 0;
  for (int i = 0; i < G && !err; ++i)
    if (x[i] < 0 || x[i] >= V) err = REF_ERR_TOKEN;
  for (int i = 0; i <= G && !err; ++i) {
    load_row(J->target, J->dtype, trow0 + i, V, zt);
    if (!row_is_valid(zt, V)) err = REF_ERR_ROW;
  }
  if (!greedy) {
    for (int i = 0; i < G && !err; ++i) {
      load_row(J->draft, J->dtype, drow0 + i, V, zd);
      if (!row_is_valid(zd, V)) err = REF_ERR_ROW;
    }
    for (int i = 0; i < G && !err; ++i) {
      float u = J->u_accept[(size_t)b * G + i];
      if (!(u >= 0.0f && u < 1.0f)) err = REF_ERR_UNIFORM;
    }
    if (!err) {
      float u = J->u_sample[b];
      if (!(u >= 0.0f && u < 1.0f)) err = REF_ERR_UNIFORM;
    }
    for (int i = 0; i < G && !err; ++i) {
      load_row(J->draft, J->dtype, drow0 + i, V, zd);
      policy(zd, V, J->T, J->k, keep_d, NULL);
      if (!keep_d[x[i]]) err = REF_ERR_QZERO;
    }
  }
  if (err) {
    J->accepted_len[b] = err;
    fill_tokens(out, G + 1, -1);
    return;
  }

  /* Chain verification ([WY] "从单个 token 接到一段 draft"; [WC] "两模型精确采样";
   * [TL] "算法"): test positions in order, stop at the first rejection. */
  for (int i = 0; i < G; ++i) {
    load_row(J->target, J->dtype, trow0 + i, V, zt);
    if (greedy) {
      int a = argmax_lowest(zt, V);
      if (x[i] == a) {
        out[i] = x[i];
        continue;
      }
      out[i] = a; /* greedy correction: the target's own choice */
      J->accepted_len[b] = i;
      fill_tokens(out + i + 1, G - i, -1);
      return;
    }
    load_row(J->draft, J->dtype, drow0 + i, V, zd);
    double logZp = policy(zt, V, J->T, J->k, keep_t, P);
    double logZq = policy(zd, V, J->T, J->k, keep_d, Q);
    /* alpha = min(1, p(x)/q(x)) ([WY] "一次 sampling 怎么执行" step 3), in log form (R7). */
    double u = (double)J->u_accept[(size_t)b * G + i];
    int accept;
    if (keep_t[x[i]]) {
      double log_px = zt[x[i]] / J->T - logZp;
      double log_qx = zd[x[i]] / J->T - logZq;
      double alpha = exp(fmin(0.0, log_px - log_qx));
      accept = (u <= alpha); /* R1 */
      if (J->accept_margin) J->accept_margin[(size_t)b * G + i] = u - alpha;
    } else {
      accept = 0; /* p(x) = 0: never emitted ([WC] reference, third assert) */
      if (J->accept_margin) J->accept_margin[(size_t)b * G + i] = INFINITY;
    }
    if (accept) {
      out[i] = x[i];
      continue;
    }
    /* Rejection: draw from norm([p - q]_+) ([WY] "Correction 为什么用正残差"; [WC]). */
    for (int v = 0; v < V; ++v) W[v] = fmax(P[v] - Q[v], 0.0);
    double d = 0.0;
    int y = ref_invcdf(W, V, (double)J->u_sample[b], &d);
    if (y < 0) y = ref_invcdf(P, V, (double)J->u_sample[b], &d); /* R4 */
    out[i] = y;
    if (J->sample_margin) J->sample_margin[b] = d;
    J->accepted_len[b] = i;
    fill_tokens(out + i + 1, G - i, -1);
    return;
  }

  /* Every draft accepted: bonus token from the target's next distribution
   * ([WY] "从单个 token 接到一段 draft"; [TL] "算法", last position). */
  load_row(J->target, J->dtype, trow0 + G, V, zt);
  if (greedy) {
    out[G] = argmax_lowest(zt, V);
  } else {
    policy(zt, V, J->T, J->k, NULL, P);
    double d = 0.0;
    out[G] = ref_invcdf(P, V, (double)J->u_sample[b], &d);
    if (J->sample_margin) J->sample_margin[b] = d;
  }
  J->accepted_len[b] = G;
}

/* ---- exported entry points -------------------------------------------------- */

/* Batched verification.  Host pointers, row-major:
 *   target [B, G+1, V], draft [B, G, V] (unused when T == 0), tokens [B, G],
 *   u_accept [B, G], u_sample [B] (unused when T == 0);
 *   outputs accepted_len [B], out_tokens [B, G+1];
 *   optional row_logz [B, 2G+1] (target rows then draft rows; NaN for invalid rows),
 *   accept_margin [B, G] (u - alpha where evaluated, else NaN; +inf when p(x) = 0),
 *   sample_margin [B] (boundary distance of the final draw; NaN if none).
 * Returns 0, or -1 for arguments it cannot process. */
int ref_spec_verify(const void *target, const void *draft, int dtype, const int32_t *tokens,
                    const float *u_accept, const float *u_sample, int B, int G, int V,
                    double temperature, int top_k, int32_t *accepted_len, int32_t *out_tokens,
                    double *row_logz, double *accept_margin, double *sample_margin,
                    int nthreads) {
  if (B < 1 || G < 0 || V < 1 || !(temperature >= 0.0) || !isfinite(temperature)) return -1;
  if (dtype != REF_F32 && dtype != REF_BF16) return -1;
  job_t J = {target, draft, dtype, tokens, u_accept, u_sample, B, G, V, temperature, top_k,
             accepted_len, out_tokens, row_logz, accept_margin, sample_margin};
  if (nthreads < 1) nthreads = 1;
#pragma omp parallel num_threads(nthreads)
  {
    double *zt = (double *)malloc(sizeof(double) * (size_t)V);
    double *zd = (double *)malloc(sizeof(double) * (size_t)V);
    double *P = (double *)malloc(sizeof(double) * (size_t)V);
    double *Q = (double *)malloc(sizeof(double) * (size_t)V);
    double *W = (double *)malloc(sizeof(double) * (size_t)V);
    unsigned char *kt = (unsigned char *)malloc((size_t)V);
    unsigned char *kd = (unsigned char *)malloc((size_t)V);
#pragma omp for schedule(dynamic, 1)
    for (int b = 0; b < B; ++b) verify_sequence(&J, b, zt, zd, P, Q, W, kt, kd);
    free(zt); free(zd); free(P); free(Q); free(W); free(kt); free(kd);
  }
  return 0;
}

/* Policy of R rows: P [R, V] probabilities (T > 0) and logz [R] log-partitions;
 * rows that are invalid get NaN.  For T == 0, P is one-hot at the lowest argmax. */
int ref_policy_rows(const void *logits, int dtype, int R, int V, double temperature, int top_k,
                    double *P, double *logz) {
  if (R < 0 || V < 1 || !(temperature >= 0.0)) return -1;
  double *z = (double *)malloc(sizeof(double) * (size_t)V);
  for (int r = 0; r < R; ++r) {
    load_row(logits, dtype, (size_t)r, V, z);
    double *Pr = P ? P + (size_t)r * V : NULL;
    if (!row_is_valid(z, V)) {
      if (Pr)
        for (int v = 0; v < V; ++v) Pr[v] = NAN;
      if (logz) logz[r] = NAN;
      continue;
    }
    if (temperature == 0.0) {
      int a = argmax_lowest(z, V);
      if (Pr)
        for (int v = 0; v < V; ++v) Pr[v] = (v == a) ? 1.0 : 0.0;
      if (logz) logz[r] = NAN;
    } else {
      double L = policy(z, V, temperature, top_k, NULL, Pr);
      if (logz) logz[r] = L;
    }
  }
  free(z);
  return 0;
}

/* Draw one token per row from the row's policy with the given uniform, by the same
 * inverse CDF ([WY] step 1: the draft's own draw X ~ q; the same draw is plain decoding
 * from p).  T == 0 gives the lowest-index argmax and reads no uniform.  Invalid rows
 * give -1 with status -3; with T > 0, a uniform outside [0,1) gives -1 with status -4
 * (the row is checked first, as in the chain).  status and margin (the draw's boundary
 * distance, 0 when none applies) may be NULL. */
int ref_sample_rows(const void *logits, int dtype, int R, int V, double temperature, int top_k,
                    const float *u, int32_t *tokens, int32_t *status, double *margin,
                    int nthreads) {
  if (R < 0 || V < 1 || !(temperature >= 0.0)) return -1;
  if (nthreads < 1) nthreads = 1;
#pragma omp parallel num_threads(nthreads)
  {
    double *z = (double *)malloc(sizeof(double) * (size_t)V);
    double *P = (double *)malloc(sizeof(double) * (size_t)V);
#pragma omp for schedule(dynamic, 4)
    for (int r = 0; r < R; ++r) {
      int32_t tok = -1, st = 0;
      double d = 0.0;
      load_row(logits, dtype, (size_t)r, V, z);
      if (!row_is_valid(z, V)) {
        st = -3;
      } else if (temperature == 0.0) {
        tok = argmax_lowest(z, V);
      } else if (!(u[r] >= 0.0f && u[r] < 1.0f)) {
        st = -4;
      } else {
        policy(z, V, temperature, top_k, NULL, P);
        tok = ref_invcdf(P, V, (double)u[r], &d);
      }
      tokens[r] = tok;
      if (status) status[r] = st;
      if (margin) margin[r] = d;
    }
    free(z);
    free(P);
  }
  return 0;
}

/* k-th largest stored logit of each row (R5), as double; NaN when top-k is inactive. */
int ref_topk_threshold_rows(const void *logits, int dtype, int R, int V, int top_k, double *tau) {
  double *z = (double *)malloc(sizeof(double) * (size_t)V);
  for (int r = 0; r < R; ++r) {
    load_row(logits, dtype, (size_t)r, V, z);
    tau[r] = topk_active(V, top_k) ? ref_topk_threshold_d(z, V, top_k) : NAN;
  }
  free(z);
  return 0;
}

/* Lowest-index argmax of each row (R6). */
int ref_argmax_rows(const void *logits, int dtype, int R, int V, int32_t *idx) {
  double *z = (double *)malloc(sizeof(double) * (size_t)V);
  for (int r = 0; r < R; ++r) {
    load_row(logits, dtype, (size_t)r, V, z);
    idx[r] = argmax_lowest(z, V);
  }
  free(z);
  return 0;
}

/* ---- overlap of every drafted position -------------------------------------- */

/* For each sequence b and position i, the two distributions the verification compares
 * there, p_i (target row i) and q_i (draft row i), after the same policy (R5, R15):
 *   beta = sum_v min(p_v, q_v)   -- the acceptance probability of the position, which is
 *          also the overlap mass ("Speculative Decoding 的朴素思想", section
 *          "为什么接受概率恰好是这个比值"; DSpark's confidence label c* and the LK loss
 *          -log beta on "推测解码：接受规则、状态与收益边界");
 *   tv   = sum_v max(p_v - q_v, 0) -- the residual mass Z, which for normalised
 *          distributions is the total variation distance, 1 - beta.
 * Both sums run in increasing v.  target holds target_rows rows per sequence (G or G+1),
 * draft G.  A pair with an unusable row (NaN, +inf, or no finite logit) gives NaN and
 * status -3, otherwise status 0.  Returns -1 for arguments it cannot process. */
int ref_overlap(const void *target, const void *draft, int dtype, int B, int G, int V,
                int target_rows, double temperature, int top_k, double *beta, double *tv,
                int32_t *status, int nthreads) {
  if (B < 0 || G < 0 || V < 1 || !(temperature > 0.0) || target_rows < G) return -1;
  if (nthreads < 1) nthreads = 1;
  const int npairs = B * G;
#pragma omp parallel num_threads(nthreads)
  {
    double *zt = (double *)malloc(sizeof(double) * (size_t)V);
    double *zd = (double *)malloc(sizeof(double) * (size_t)V);
    double *P = (double *)malloc(sizeof(double) * (size_t)V);
    double *Q = (double *)malloc(sizeof(double) * (size_t)V);
#pragma omp for schedule(dynamic, 2)
    for (int n = 0; n < npairs; ++n) {
      const int b = n / G, i = n - b * G;
      load_row(target, dtype, (size_t)b * target_rows + i, V, zt);
      load_row(draft, dtype, (size_t)b * G + i, V, zd);
      if (!row_is_valid(zt, V) || !row_is_valid(zd, V)) {
        beta[n] = NAN;
        tv[n] = NAN;
        if (status) status[n] = REF_ERR_ROW;
        continue;
      }
      policy(zt, V, temperature, top_k, NULL, P);
      policy(zd, V, temperature, top_k, NULL, Q);
      double sb = 0.0, st = 0.0;
      for (int v = 0; v < V; ++v) {
        sb += fmin(P[v], Q[v]);
        st += fmax(P[v] - Q[v], 0.0);
      }
      beta[n] = sb;
      tv[n] = st;
      if (status) status[n] = 0;
    }
    free(zt);
    free(zd);
    free(P);
    free(Q);
  }
  return 0;
}

/* ---- tree verification (R16) ----------------------------------------------------- */

/* Batched tree verification.  Host pointers, row-major:
 *   target, draft [B, N, V] logits (draft rows of leaves are not read), tokens, parent
 *   [B, N] int32 (node 0: the root, parent -1, token unused), u_accept [B, N] (node n's
 *   test uses u_accept[b, n]), u_sample [B].  Outputs: accepted_len [B] (the depth of
 *   the accepted path, or a negative code), out_tokens [B, N] (the accepted tokens, then
 *   the correction or bonus token, then -1), path_nodes [B, N] (the accepted nodes, then
 *   -1; nullable), accept_margin [B, N] (u - alpha of each tested node, NaN for untested
 *   ones, +inf when p(x) = 0; nullable), sample_margin [B] (nullable).
 * Checks, in this order: the tree (-6), tokens (-1), the rows the walk may read (-3), the
 * uniforms (-4), q_parent(x_n) > 0 for every node (-2).  Returns -1 for arguments it
 * cannot process. */
int ref_tree_verify(const void *target, const void *draft, int dtype, const int32_t *tokens,
                    const int32_t *parent, const float *u_accept, const float *u_sample, int B,
                    int N, int V, double T, int top_k, int32_t *accepted_len,
                    int32_t *out_tokens, int32_t *path_nodes, double *accept_margin,
                    double *sample_margin, int nthreads) {
  if (B < 0 || N < 1 || V < 1 || !(T >= 0.0)) return -1;
  if (nthreads < 1) nthreads = 1;
  const int greedy = (T == 0.0);
#pragma omp parallel num_threads(nthreads)
  {
    double *zt = (double *)malloc(sizeof(double) * (size_t)V);
    double *zd = (double *)malloc(sizeof(double) * (size_t)V);
    double *P = (double *)malloc(sizeof(double) * (size_t)V);
    double *Q = (double *)malloc(sizeof(double) * (size_t)V);
    double *cur = (double *)malloc(sizeof(double) * (size_t)V);
    unsigned char *keep_t = (unsigned char *)malloc((size_t)V);
    unsigned char *keep_d = (unsigned char *)malloc((size_t)V);
    int *nchild = (int *)malloc(sizeof(int) * (size_t)N);
#pragma omp for schedule(dynamic, 1)
    for (int b = 0; b < B; ++b) {
      const int32_t *par = parent + (size_t)b * N;
      const int32_t *x = tokens + (size_t)b * N;
      const size_t row0 = (size_t)b * N;
      int32_t *out = out_tokens + (size_t)b * N;
      int32_t *path = path_nodes ? path_nodes + (size_t)b * N : NULL;
      fill_tokens(out, N, -1);
      if (path) fill_tokens(path, N, -1);
      if (accept_margin)
        for (int n = 0; n < N; ++n) accept_margin[row0 + n] = NAN;
      if (sample_margin) sample_margin[b] = NAN;

      int err = 0;
      if (par[0] != -1) err = REF_ERR_TREE;
      for (int n = 1; n < N && !err; ++n)
        if (par[n] < 0 || par[n] >= n) err = REF_ERR_TREE;
      for (int n = 0; n < N; ++n) nchild[n] = 0;
      if (!err)
        for (int n = 1; n < N; ++n) nchild[par[n]]++;
      for (int n = 1; n < N && !err; ++n)
        if (x[n] < 0 || x[n] >= V) err = REF_ERR_TOKEN;
      for (int n = 0; n < N && !err; ++n) {
        load_row(target, dtype, row0 + n, V, zt);
        if (!row_is_valid(zt, V)) err = REF_ERR_ROW;
      }
      if (!greedy) {
        for (int n = 0; n < N && !err; ++n) {
          if (!nchild[n]) continue;
          load_row(draft, dtype, row0 + n, V, zd);
          if (!row_is_valid(zd, V)) err = REF_ERR_ROW;
        }
        for (int n = 1; n < N && !err; ++n) {
          float u = u_accept[row0 + n];
          if (!(u >= 0.0f && u < 1.0f)) err = REF_ERR_UNIFORM;
        }
        if (!err && !(u_sample[b] >= 0.0f && u_sample[b] < 1.0f)) err = REF_ERR_UNIFORM;
        for (int n = 1; n < N && !err; ++n) {
          load_row(draft, dtype, row0 + par[n], V, zd);
          policy(zd, V, T, top_k, keep_d, NULL);
          if (!keep_d[x[n]]) err = REF_ERR_QZERO;
        }
      }
      if (err) {
        accepted_len[b] = err;
        continue;
      }

      int u = 0, depth = 0;
      for (;;) {
        load_row(target, dtype, row0 + u, V, zt);
        if (greedy) {
          int a = argmax_lowest(zt, V), next = -1;
          for (int s = u + 1; s < N && next < 0; ++s)
            if (par[s] == u && x[s] == a) next = s;
          out[depth] = a;
          if (next < 0) break; /* the target's own choice ends the round */
          if (path) path[depth] = next;
          ++depth;
          u = next;
          continue;
        }
        double logZp = policy(zt, V, T, top_k, keep_t, P);
        if (!nchild[u]) { /* a leaf: bonus from p_u */
          double d = 0.0;
          out[depth] = ref_invcdf(P, V, (double)u_sample[b], &d);
          if (sample_margin) sample_margin[b] = d;
          break;
        }
        load_row(draft, dtype, row0 + u, V, zd);
        double logZq = policy(zd, V, T, top_k, keep_d, Q);
        for (int v = 0; v < V; ++v) cur[v] = P[v];
        int rejected = 0, next = -1;
        for (int s = u + 1; s < N && next < 0; ++s) {
          if (par[s] != u) continue;
          const int xs = x[s];
          const double us = (double)u_accept[row0 + s];
          double alpha;
          if (!rejected) { /* the first child: min(1, p/q) as in the chain (R7) */
            alpha = keep_t[xs] ? exp(fmin(0.0, (zt[xs] / T - logZp) - (zd[xs] / T - logZq))) : 0.0;
          } else {         /* later siblings: the current residual distribution */
            alpha = fmin(1.0, cur[xs] / Q[xs]);
          }
          const int has_p = rejected ? (cur[xs] > 0.0) : keep_t[xs];
          if (accept_margin) accept_margin[row0 + s] = has_p ? us - alpha : INFINITY;
          if (has_p && us <= alpha) { /* R1 */
            next = s;
            break;
          }
          /* rejected: cur <- norm([cur - q_u]_+) before the next sibling */
          double Z = 0.0;
          for (int v = 0; v < V; ++v) Z += fmax(cur[v] - Q[v], 0.0);
          if (Z > 0.0)
            for (int v = 0; v < V; ++v) cur[v] = fmax(cur[v] - Q[v], 0.0) / Z;
          else /* zero mass (as R4): p_u is the current distribution again */
            for (int v = 0; v < V; ++v) cur[v] = P[v];
          ++rejected;
        }
        if (next < 0) { /* every child rejected: draw from the current distribution */
          double d = 0.0;
          out[depth] = ref_invcdf(cur, V, (double)u_sample[b], &d);
          if (sample_margin) sample_margin[b] = d;
          break;
        }
        out[depth] = x[next];
        if (path) path[depth] = next;
        ++depth;
        u = next;
      }
      accepted_len[b] = depth;
    }
    free(zt);
    free(zd);
    free(P);
    free(Q);
    free(cur);
    free(keep_t);
    free(keep_d);
    free(nchild);
  }
  return 0;
}

/* ---- typical acceptance (R17) --------------------------------------------------- */

/* Entropy in nats of the policy distribution P (terms with P = 0 contribute 0). */
static double entropy(const double *P, int V) {
  double h = 0.0;
  for (int v = 0; v < V; ++v)
    if (P[v] > 0.0) h -= P[v] * log(P[v]);
  return h;
}

/* Batched typical acceptance.  target [B, G+1, V], tokens [B, G]; T > 0.  Outputs
 * accepted_len [B] (0..G, or -1 token outside [0,V) / -3 an unusable target row, checked
 * in that order over all positions) and out_tokens [B, G+1] (the accepted drafts, then
 * argmax p_{j+1}, then -1).  margin [B, G] (nullable): log p_i(x_i) - log(threshold) of
 * every position, +inf where the threshold is 0, NaN where not formed.  entropy_out [B,
 * G+1] (nullable): H of every target row.  Returns -1 for arguments it cannot process. */
int ref_typical_verify(const void *target, int dtype, const int32_t *tokens, int B, int G, int V,
                       double T, int top_k, double eps, double delta, int32_t *accepted_len,
                       int32_t *out_tokens, double *margin, double *entropy_out, int nthreads) {
  if (B < 0 || G < 0 || V < 1 || !(T > 0.0) || !(eps >= 0.0) || !(delta >= 0.0)) return -1;
  if (nthreads < 1) nthreads = 1;
#pragma omp parallel num_threads(nthreads)
  {
    double *z = (double *)malloc(sizeof(double) * (size_t)V);
    double *P = (double *)malloc(sizeof(double) * (size_t)V);
#pragma omp for schedule(dynamic, 1)
    for (int b = 0; b < B; ++b) {
      const int32_t *x = tokens + (size_t)b * G;
      int32_t *out = out_tokens + (size_t)b * (G + 1);
      const size_t row0 = (size_t)b * (G + 1);
      if (margin)
        for (int i = 0; i < G; ++i) margin[(size_t)b * G + i] = NAN;
      if (entropy_out)
        for (int i = 0; i <= G; ++i) entropy_out[row0 + i] = NAN;
      int err = 0;
      for (int i = 0; i < G && !err; ++i)
        if (x[i] < 0 || x[i] >= V) err = REF_ERR_TOKEN;
      for (int i = 0; i <= G && !err; ++i) {
        load_row(target, dtype, row0 + i, V, z);
        if (!row_is_valid(z, V)) err = REF_ERR_ROW;
      }
      if (err) {
        accepted_len[b] = err;
        fill_tokens(out, G + 1, -1);
        continue;
      }
      if (entropy_out)
        for (int i = 0; i <= G; ++i) {
          load_row(target, dtype, row0 + i, V, z);
          policy(z, V, T, top_k, NULL, P);
          entropy_out[row0 + i] = entropy(P, V);
        }
      int j = G;
      for (int i = 0; i < G; ++i) {
        load_row(target, dtype, row0 + i, V, z);
        policy(z, V, T, top_k, NULL, P);
        const double H = entropy(P, V);
        const double thr = fmin(eps, delta * exp(-H));
        const double px = P[x[i]];
        if (margin) margin[(size_t)b * G + i] = (thr > 0.0) ? log(px) - log(thr) : INFINITY;
        if (!(px > thr)) { /* the first position that is not typical ends the prefix */
          j = i;
          break;
        }
      }
      for (int i = 0; i < j; ++i) out[i] = x[i];
      load_row(target, dtype, row0 + j, V, z);
      out[j] = argmax_lowest(z, V); /* the next token: the target's greedy choice */
      fill_tokens(out + j + 1, G - j, -1);
      accepted_len[b] = j;
    }
    free(z);
    free(P);
  }
  return 0;
}
