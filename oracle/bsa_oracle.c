/*
 * bsa_oracle.c -- plain, slow, single-threaded fp64 CPU oracle for block-sparse
 * attention with summary-based block routing.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call this code:
 * only the test suite, the smoke check and the benchmark's CPU-baseline leg use
 * it.  It shares no code, header, table or helper with the HIP library.
 *
 * Every step follows the pages' statement of the method, in their order:
 *   - "DashAttention", section "Estágio 0: Resumo de Blocos Locais": the
 *     context is split into contiguous blocks of size B and each block is
 *     compressed into one key summary by a learned query that, initialised at
 *     zero, reduces to uniform mean pooling; a summary is fixed once its block
 *     is complete.
 *   - "DashAttention", section "Estágio 1: Roteamento de Blocos via Entmax"
 *     (equation w = alpha-entmax(gamma z)) and the "Declaração do Problema"
 *     (top-k block selection from coarse scores followed by fine softmax over
 *     the selected tokens); GQA heads average their routing probabilities.
 *   - "DashAttention", section "Estágio 2": the diagonal block is handled by a
 *     separate branch (always attended).
 *   - "AdaSplash-2", section 2.A: a 16-bin histogram of the scores on the unit
 *     interval gives a provable lower bound for the entmax threshold tau,
 *     refined by a root finder (here: bisection, at most max_iter steps).
 *   - "Gist Sparse Attention", section 2 item 3: the k most relevant blocks
 *     are unfolded into their raw tokens for exact attention.
 *
 * Numerics: inputs are fp32 arrays (bf16 data is upcast exactly by the caller);
 * every sum, product, exp, pow and sqrt is done in double with the host libm.
 * No BLAS, no threads, no -ffast-math.
 *
 * Parity pins: every function here is pinned by the CPU tests (closed forms,
 * brute force, library routines, invariants).  See the test files for which
 * pin covers which function.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_FORCE_DIAG 1u
#define ORC_FORCE_FIRST 2u
#define ORC_FORCE_TAIL 4u

#define ORC_MODE_PREFILL 0
#define ORC_MODE_DECODE 1
#define ORC_MODE_TOKEN 2 /* causal prefill routed per query token */

const char *orc_version(void) { return "bsa-oracle 1"; }

/* ------------------------------------------------------------------------- */
/* Stage 0: block summaries.                                                  */
/* ------------------------------------------------------------------------- */

/*
 * Key summary of every block ("DashAttention", Estágio 0).
 *   K    : [nb, nh, n, d] row-major fp32.
 *   qbar : NULL -> zero learned query -> uniform mean of the block's keys.
 *          else [nh, d]: weights w_t = softmax_t(qbar . k_t / sqrt(d)) over the
 *          block's keys, summary = sum_t w_t k_t (local scaled dot-product
 *          attention of the learned query over the block).
 *   S    : [nb, nh, nblk, d] fp64, nblk = ceil(n / B).  A trailing partial
 *          block uses only the tokens present.
 */
void orc_summarize(const float *K, int64_t nb, int64_t nh, int64_t n, int64_t d,
                   int64_t B, const float *qbar, double *S) {
  int64_t nblk = (n + B - 1) / B;
  double *w = (double *)malloc(sizeof(double) * (size_t)B);
  for (int64_t b = 0; b < nb; ++b)
    for (int64_t h = 0; h < nh; ++h)
      for (int64_t j = 0; j < nblk; ++j) {
        int64_t t0 = j * B;
        int64_t t1 = t0 + B < n ? t0 + B : n;
        int64_t cntj = t1 - t0;
        const float *kb = K + ((b * nh + h) * n) * d;
        double *s = S + ((b * nh + h) * nblk + j) * d;
        if (qbar == NULL) {
          for (int64_t t = 0; t < cntj; ++t) w[t] = 1.0 / (double)cntj;
        } else {
          const float *qb = qbar + h * d;
          double mx = -INFINITY;
          for (int64_t t = 0; t < cntj; ++t) {
            double a = 0.0;
            for (int64_t c = 0; c < d; ++c)
              a += (double)qb[c] * (double)kb[(t0 + t) * d + c];
            a /= sqrt((double)d);
            w[t] = a;
            if (a > mx) mx = a;
          }
          double z = 0.0;
          for (int64_t t = 0; t < cntj; ++t) {
            w[t] = exp(w[t] - mx);
            z += w[t];
          }
          for (int64_t t = 0; t < cntj; ++t) w[t] /= z;
        }
        for (int64_t c = 0; c < d; ++c) {
          double acc = 0.0;
          for (int64_t t = 0; t < cntj; ++t) acc += w[t] * (double)kb[(t0 + t) * d + c];
          s[c] = acc;
        }
      }
  free(w);
}

/*
 * Routing query of each query block: the mean of the block's queries, per
 * head.  With a single query token (decode) this is the query itself.
 *   Q    : [nb, nh, n, d] fp32.   qhat : [nb, nh, ceil(n/B), d] fp64.
 */
void orc_qpool(const float *Q, int64_t nb, int64_t nh, int64_t n, int64_t d, int64_t B,
               double *qhat) {
  int64_t nblk = (n + B - 1) / B;
  for (int64_t b = 0; b < nb; ++b)
    for (int64_t h = 0; h < nh; ++h)
      for (int64_t i = 0; i < nblk; ++i) {
        int64_t t0 = i * B;
        int64_t t1 = t0 + B < n ? t0 + B : n;
        const float *qb = Q + ((b * nh + h) * n) * d;
        double *o = qhat + ((b * nh + h) * nblk + i) * d;
        for (int64_t c = 0; c < d; ++c) {
          double acc = 0.0;
          for (int64_t t = t0; t < t1; ++t) acc += (double)qb[t * d + c];
          o[c] = acc / (double)(t1 - t0);
        }
      }
}

/* ------------------------------------------------------------------------- */
/* Shared routing bookkeeping: which blocks are candidates, which are forced. */
/* ------------------------------------------------------------------------- */

/*
 * For one routing row, returns the candidate range [0, cand_end) of blocks
 * that may be scored and the list of forced blocks.
 *   prefill (row = query block i): top-k candidates are the blocks j <= i
 *     (causal; the diagonal may win on score); entmax candidates are j < i,
 *     because the diagonal is the separate always-attended branch.
 *     DIAG forces i, FIRST forces 0; TAIL has no meaning in prefill.
 *   decode (row = one query at position L-1): the query's own block
 *     tail = floor((L-1)/B) is incomplete and has no summary, so candidates are
 *     the complete blocks j < tail; TAIL (and DIAG, its synonym) forces the
 *     tail block, FIRST forces block 0.
 *   token (row = query position t of a causal prefill, routed on its own as
 *     "DashAttention", Estágio 1 routes each query): as prefill with the
 *     query's own block t / B in place of the query block.
 * Forced blocks are removed from the candidate set by the callers.
 */
static int64_t row_setup(int mode, int entmax, int64_t row, int64_t kv_len, int64_t B,
                         uint32_t force, int64_t *forced, int *nforced) {
  int64_t own, cand_end;
  if (mode == ORC_MODE_PREFILL || mode == ORC_MODE_TOKEN) {
    own = mode == ORC_MODE_TOKEN ? row / B : row;
    cand_end = entmax ? own : own + 1;
  } else {
    own = (kv_len - 1) / B;
    cand_end = own;
  }
  int nf = 0;
  int64_t list[3];
  if (force & ORC_FORCE_FIRST) list[nf++] = 0;
  if ((force & ORC_FORCE_DIAG) || (mode == ORC_MODE_DECODE && (force & ORC_FORCE_TAIL)))
    list[nf++] = own;
  /* dedupe (first == own when own == 0) */
  *nforced = 0;
  for (int a = 0; a < nf; ++a) {
    int dup = 0;
    for (int c = 0; c < *nforced; ++c)
      if (forced[c] == list[a]) dup = 1;
    if (!dup) forced[(*nforced)++] = list[a];
  }
  return cand_end;
}

static int is_forced(int64_t j, const int64_t *forced, int nforced) {
  for (int a = 0; a < nforced; ++a)
    if (forced[a] == j) return 1;
  return 0;
}

/* Order by score descending, then block index ascending (lower index wins ties). */
typedef struct {
  double key;
  int64_t j;
} keyed_t;

static int cmp_keyed_desc(const void *pa, const void *pb) {
  const keyed_t *a = (const keyed_t *)pa, *b = (const keyed_t *)pb;
  if (a->key > b->key) return -1;
  if (a->key < b->key) return 1;
  return (a->j < b->j) ? -1 : (a->j > b->j) ? 1 : 0;
}

static int cmp_i64(const void *pa, const void *pb) {
  int64_t a = *(const int64_t *)pa, b = *(const int64_t *)pb;
  return (a < b) ? -1 : (a > b) ? 1 : 0;
}

/* ------------------------------------------------------------------------- */
/* Stage 1a: top-k routing.                                                    */
/* ------------------------------------------------------------------------- */

/*
 * Top-k block routing over summary scores ("DashAttention", Declaração do
 * Problema: top-k KV blocks from coarse scores; "Gist Sparse Attention",
 * section 2 item 3: select the k most relevant blocks).
 *
 *   qhat   : [nb, hq, nrow, d]  routing queries per query head.
 *   S      : [nb, hkv, nblk, d] block summaries.
 *   Score of block j for the row of KV head g:
 *            (1/sqrt(d)) * sum over the query heads h of group g of qhat_h . s_j
 *            (heads grouped contiguously: g(h) = h / (hq/hkv)).
 *   kv_lens: decode only, [nb] current lengths L (query at position L-1).
 *   k_total: total selected blocks per row, forced ones included.
 *   Outputs, per (b, g, row):
 *     idx   [.., k_total] ascending block ids, -1 padded;  cnt [..].
 *     scores[.., nblk] (may be NULL): candidate scores, -inf elsewhere.
 *     gap   [..] (may be NULL): (m-th best) - (m+1-th best) routed candidate
 *           score, +inf when the routed set is forced by the count alone.
 */
void orc_route_topk(const double *qhat, const double *S, int64_t nb, int64_t hq, int64_t hkv,
                    int64_t nrow, int64_t nblk, int64_t d, int64_t B, int mode,
                    const int64_t *kv_lens, int64_t k_total, uint32_t force, double score_scale,
                    int32_t *idx, int32_t *cnt, double *scores, double *gap) {
  int64_t G = hq / hkv;
  keyed_t *cand = (keyed_t *)malloc(sizeof(keyed_t) * (size_t)(nblk + 1));
  int64_t *sel = (int64_t *)malloc(sizeof(int64_t) * (size_t)(k_total + 3));
  double *sc = (double *)malloc(sizeof(double) * (size_t)(nblk + 1));
  for (int64_t b = 0; b < nb; ++b)
    for (int64_t g = 0; g < hkv; ++g)
      for (int64_t r = 0; r < nrow; ++r) {
        int64_t forced[3];
        int nforced = 0;
        int64_t L = (mode == ORC_MODE_DECODE) ? kv_lens[b] : 0;
        int64_t cend = row_setup(mode, 0, r, L, B, force, forced, &nforced);
        int64_t rowid = (b * hkv + g) * nrow + r;
        /* scores of every candidate block */
        for (int64_t j = 0; j < nblk; ++j) sc[j] = -INFINITY;
        for (int64_t j = 0; j < cend; ++j) {
          double acc = 0.0;
          for (int64_t h = g * G; h < (g + 1) * G; ++h) {
            const double *qv = qhat + ((b * hq + h) * nrow + r) * d;
            const double *sv = S + ((b * hkv + g) * nblk + j) * d;
            double dot = 0.0;
            for (int64_t c = 0; c < d; ++c) dot += qv[c] * sv[c];
            acc += dot;
          }
          sc[j] = acc * score_scale;
        }
        if (scores)
          for (int64_t j = 0; j < nblk; ++j) scores[rowid * nblk + j] = sc[j];
        /* the routed candidates exclude the forced blocks */
        int64_t nc = 0;
        for (int64_t j = 0; j < cend; ++j)
          if (!is_forced(j, forced, nforced)) {
            cand[nc].key = sc[j];
            cand[nc].j = j;
            ++nc;
          }
        int64_t m = k_total - nforced;
        if (m < 0) m = 0;
        qsort(cand, (size_t)nc, sizeof(keyed_t), cmp_keyed_desc);
        int64_t take = m < nc ? m : nc;
        if (gap) gap[rowid] = (m > 0 && nc > m) ? cand[m - 1].key - cand[m].key : INFINITY;
        int64_t ns = 0;
        for (int a = 0; a < nforced; ++a) sel[ns++] = forced[a];
        for (int64_t a = 0; a < take; ++a) sel[ns++] = cand[a].j;
        qsort(sel, (size_t)ns, sizeof(int64_t), cmp_i64);
        cnt[rowid] = (int32_t)ns;
        for (int64_t a = 0; a < k_total; ++a)
          idx[rowid * k_total + a] = a < ns ? (int32_t)sel[a] : -1;
      }
  free(cand);
  free(sel);
  free(sc);
}

/* ------------------------------------------------------------------------- */
/* Stage 1b: alpha-entmax routing with a histogram-initialised bisection.     */
/* ------------------------------------------------------------------------- */

/*
 * alpha-entmax in the parametrisation p_j = [x_j - tau]_+^(1/(alpha-1)) with
 * x = (alpha-1) z and tau chosen so that sum_j p_j = 1.  alpha = 2 is
 * sparsemax; alpha -> 1 tends to softmax.
 */
static double entmax_mass(const double *x, int64_t n, double tau, double alpha) {
  double e = 1.0 / (alpha - 1.0), acc = 0.0;
  for (int64_t a = 0; a < n; ++a)
    if (x[a] > tau) acc += pow(x[a] - tau, e);
  return acc;
}

/*
 * Solve sum_b c_b [e_b - tau]_+^(1/(alpha-1)) = 1 for tau, with the values e_b
 * sorted descending and integer multiplicities c_b (a histogram, or a plain
 * list with all c_b = 1).  alpha = 2 and alpha = 1.5 use the exact sort-based
 * closed forms (sparsemax: Martins & Astudillo 2016; 1.5-entmax: Peters,
 * Niculae & Martins 2019); other alpha use 64 bisection steps on
 * [e_0 - 1, e_0], where the root always lies.
 */
static double solve_sorted(const double *e, const int64_t *c, int64_t nb_, double alpha) {
  if (alpha == 2.0 || alpha == 1.5) {
    double n = 0.0, s1 = 0.0, s2 = 0.0;
    for (int64_t r = 0; r < nb_; ++r) {
      if (c[r] == 0) continue;
      n += (double)c[r];
      s1 += (double)c[r] * e[r];
      s2 += (double)c[r] * e[r] * e[r];
      double tau;
      if (alpha == 2.0) {
        tau = (s1 - 1.0) / n;
      } else {
        double M = s1 / n;
        double Q = s2 - n * M * M; /* sum of squared deviations */
        if (Q > 1.0) continue;     /* support too wide: the root is above e_r */
        tau = M - sqrt((1.0 - Q) / n);
      }
      /* next nonempty value below this prefix */
      int64_t nx = r + 1;
      while (nx < nb_ && c[nx] == 0) ++nx;
      int ok_here = tau < e[r];
      int ok_next = (nx >= nb_) || tau >= e[nx];
      if (ok_here && ok_next) return tau;
    }
    /* unreachable for well-formed input; fall through to bisection */
  }
  double lo = e[0] - 1.0, hi = e[0];
  double ex = 1.0 / (alpha - 1.0);
  for (int it = 0; it < 64; ++it) {
    double mid = 0.5 * (lo + hi), f = 0.0;
    for (int64_t r = 0; r < nb_; ++r)
      if (e[r] > mid) f += (double)c[r] * pow(e[r] - mid, ex);
    if (f >= 1.0)
      lo = mid;
    else
      hi = mid;
  }
  return 0.5 * (lo + hi);
}

static int cmp_dbl_desc(const void *pa, const void *pb) {
  double a = *(const double *)pa, b = *(const double *)pb;
  return (a > b) ? -1 : (a < b) ? 1 : 0;
}

/*
 * Threshold tau of one entmax row by the histogram-started bisection
 * ("AdaSplash-2", sections 2.A and 1).  Returns tau; *resolved tells whether
 * the support was pinned down exactly, *iters counts bisection steps and
 * tlo and thi receive the histogram bracket.
 *
 *   1. x_max = max x.
 *   2. Histogram of u = x_max - x on the unit interval with n_bins bins
 *      (values with u >= 1 can never be in the support, since tau >= x_max-1).
 *   3. tau_lo solves the problem with every value moved to its bin's lower edge
 *      (x_max - (b+1)/n_bins): a lower bound on tau.  tau_hi uses upper edges
 *      (x_max - b/n_bins): an upper bound.
 *   4. lo = max(tau_lo, x_max - 1), hi = min(tau_hi, x_max - n^(1-alpha)).
 *   5. Up to max_iter times: stop when no x lies in (lo, hi] (support
 *      resolved); else bisect on the exact mass.
 *   6. Resolved: tau is the exact threshold of the support {x > lo}.
 *      Otherwise tau = lo (a superset support).
 */
static double entmax_tau(const double *x, int64_t n, double alpha, int n_bins, int max_iter,
                         int *resolved, int *iters, double *tlo, double *thi) {
  double xmax = -INFINITY;
  for (int64_t a = 0; a < n; ++a)
    if (x[a] > xmax) xmax = x[a];
  int64_t *cnts = (int64_t *)calloc((size_t)n_bins, sizeof(int64_t));
  double *edge = (double *)malloc(sizeof(double) * (size_t)n_bins);
  for (int64_t a = 0; a < n; ++a) {
    double u = xmax - x[a];
    if (u < 1.0) {
      int64_t bin = (int64_t)floor(u * (double)n_bins);
      if (bin > n_bins - 1) bin = n_bins - 1;
      cnts[bin] += 1;
    }
  }
  for (int b = 0; b < n_bins; ++b) edge[b] = xmax - (double)(b + 1) / (double)n_bins;
  double tau_lo = solve_sorted(edge, cnts, n_bins, alpha);
  for (int b = 0; b < n_bins; ++b) edge[b] = xmax - (double)b / (double)n_bins;
  double tau_hi = solve_sorted(edge, cnts, n_bins, alpha);
  free(cnts);
  free(edge);
  if (tlo) *tlo = tau_lo;
  if (thi) *thi = tau_hi;

  double lo = tau_lo > xmax - 1.0 ? tau_lo : xmax - 1.0;
  double ub = xmax - pow((double)n, 1.0 - alpha);
  double hi = tau_hi < ub ? tau_hi : ub;
  int it = 0, res = 0;
  for (;;) {
    int inside = 0;
    for (int64_t a = 0; a < n; ++a)
      if (x[a] > lo && x[a] <= hi) {
        inside = 1;
        break;
      }
    if (!inside) {
      res = 1;
      break;
    }
    if (it >= max_iter) break;
    double mid = 0.5 * (lo + hi);
    if (entmax_mass(x, n, mid, alpha) >= 1.0)
      lo = mid;
    else
      hi = mid;
    ++it;
  }
  *iters = it;
  *resolved = res;
  if (!res) return lo;
  /* exact threshold on the resolved support {x > lo} */
  int64_t ns = 0;
  double *sup = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
  for (int64_t a = 0; a < n; ++a)
    if (x[a] > lo) sup[ns++] = x[a];
  qsort(sup, (size_t)ns, sizeof(double), cmp_dbl_desc);
  double tau;
  if (alpha == 2.0) {
    double s1 = 0.0;
    for (int64_t a = 0; a < ns; ++a) s1 += sup[a];
    tau = (s1 - 1.0) / (double)ns;
  } else if (alpha == 1.5) {
    double s1 = 0.0;
    for (int64_t a = 0; a < ns; ++a) s1 += sup[a];
    double M = s1 / (double)ns, Q = 0.0;
    for (int64_t a = 0; a < ns; ++a) Q += (sup[a] - M) * (sup[a] - M);
    double r = (1.0 - Q) / (double)ns;
    tau = M - sqrt(r > 0.0 ? r : 0.0);
  } else {
    int64_t *ones = (int64_t *)malloc(sizeof(int64_t) * (size_t)ns);
    for (int64_t a = 0; a < ns; ++a) ones[a] = 1;
    tau = solve_sorted(sup, ones, ns, alpha);
    free(ones);
  }
  free(sup);
  return tau;
}

/*
 * Exported single-row entmax for pinning: p = alpha-entmax over x (already
 * multiplied by alpha-1), via the histogram-started bisection above.
 */
double orc_entmax_row(const double *x, int64_t n, double alpha, int n_bins, int max_iter,
                      double *p, int *resolved, int *iters, double *tau_lo, double *tau_hi) {
  double tau = entmax_tau(x, n, alpha, n_bins, max_iter, resolved, iters, tau_lo, tau_hi);
  double e = 1.0 / (alpha - 1.0), z = 0.0;
  for (int64_t a = 0; a < n; ++a) {
    p[a] = x[a] > tau ? pow(x[a] - tau, e) : 0.0;
    z += p[a];
  }
  for (int64_t a = 0; a < n; ++a) p[a] /= z;
  return tau;
}

/*
 * Entmax block routing ("DashAttention", Estágio 1, with GQA averaging;
 * threshold per "AdaSplash-2" 2.A).  Per (b, query head h, row):
 *   z_j = gamma * qhat_h . s_j / sqrt(d) over the candidate blocks (forced ones
 *   excluded), x = (alpha-1) z, tau by entmax_tau, p_j = [x_j - tau]^(1/(alpha-1))
 *   renormalised.  Per KV head g: wbar_j = mean of p_j over the group's heads;
 *   the kept set is {wbar > 0}, cut to the top `cap` by (wbar desc, j asc) when
 *   larger; the selection is ascending(kept + forced).
 *
 *   idx     [nb, hkv, nrow, cap + nforce_max] ascending, -1 padded; cnt [..].
 *   probs   [nb, hq, nrow, nblk] (may be NULL): p, zero outside the candidates.
 *   tau     [nb, hq, nrow] (may be NULL).
 *   margin  [nb, hq, nrow] (may be NULL): min over candidates of |x_j - tau|
 *           (+inf without candidates).
 *   capgap  [nb, hkv, nrow] (may be NULL): wbar_(cap) - wbar_(cap+1) among
 *           nonzero wbar, +inf when the cap does not bind.
 *   resolved/iters [nb, hq, nrow] (may be NULL).
 *   wsel    [nb, hkv, nrow, idx_width] (may be NULL): the routing weight of
 *           each listed block, wbar_j for a routed block and 1 for a forced
 *           one (forced blocks have no routing score: "DashAttention",
 *           Estágio 2, the diagonal keeps a branch of its own); 0 padded.
 */
void orc_route_entmax(const double *qhat, const double *S, int64_t nb, int64_t hq, int64_t hkv,
                      int64_t nrow, int64_t nblk, int64_t d, int64_t B, int mode,
                      const int64_t *kv_lens, double alpha, double gamma, int n_bins, int max_iter,
                      int64_t cap, uint32_t force, double score_scale, int64_t idx_width,
                      int32_t *idx, int32_t *cnt, double *probs, double *tau_out, double *margin,
                      double *capgap, int32_t *resolved_out, int32_t *iters_out,
                      double *wsel) {
  int64_t G = hq / hkv;
  double *x = (double *)malloc(sizeof(double) * (size_t)(nblk + 1));
  double *p = (double *)malloc(sizeof(double) * (size_t)(nblk + 1));
  double *wbar = (double *)malloc(sizeof(double) * (size_t)(nblk + 1));
  int64_t *cj = (int64_t *)malloc(sizeof(int64_t) * (size_t)(nblk + 1));
  keyed_t *kw = (keyed_t *)malloc(sizeof(keyed_t) * (size_t)(nblk + 1));
  int64_t *sel = (int64_t *)malloc(sizeof(int64_t) * (size_t)(nblk + 4));
  for (int64_t b = 0; b < nb; ++b)
    for (int64_t g = 0; g < hkv; ++g)
      for (int64_t r = 0; r < nrow; ++r) {
        int64_t forced[3];
        int nforced = 0;
        int64_t L = (mode == ORC_MODE_DECODE) ? kv_lens[b] : 0;
        int64_t cend = row_setup(mode, 1, r, L, B, force, forced, &nforced);
        int64_t nc = 0;
        for (int64_t j = 0; j < cend; ++j)
          if (!is_forced(j, forced, nforced)) cj[nc++] = j;
        for (int64_t a = 0; a < nc; ++a) wbar[a] = 0.0;
        for (int64_t h = g * G; h < (g + 1) * G; ++h) {
          int64_t hrow = (b * hq + h) * nrow + r;
          const double *qv = qhat + hrow * d;
          for (int64_t a = 0; a < nc; ++a) {
            const double *sv = S + ((b * hkv + g) * nblk + cj[a]) * d;
            double dot = 0.0;
            for (int64_t c = 0; c < d; ++c) dot += qv[c] * sv[c];
            x[a] = (alpha - 1.0) * gamma * dot * score_scale;
          }
          double tau = NAN, mg = INFINITY;
          int res = 1, its = 0;
          if (nc > 0) {
            tau = orc_entmax_row(x, nc, alpha, n_bins, max_iter, p, &res, &its, NULL, NULL);
            for (int64_t a = 0; a < nc; ++a) {
              double dd = fabs(x[a] - tau);
              if (dd < mg) mg = dd;
              wbar[a] += p[a];
            }
          }
          if (probs) {
            for (int64_t j = 0; j < nblk; ++j) probs[hrow * nblk + j] = 0.0;
            for (int64_t a = 0; a < nc; ++a) probs[hrow * nblk + cj[a]] = p[a];
          }
          if (tau_out) tau_out[hrow] = tau;
          if (margin) margin[hrow] = mg;
          if (resolved_out) resolved_out[hrow] = res;
          if (iters_out) iters_out[hrow] = its;
        }
        int64_t rowid = (b * hkv + g) * nrow + r;
        int64_t nk = 0;
        for (int64_t a = 0; a < nc; ++a) {
          double w = wbar[a] / (double)G;
          if (w > 0.0) {
            kw[nk].key = w;
            kw[nk].j = cj[a];
            ++nk;
          }
        }
        qsort(kw, (size_t)nk, sizeof(keyed_t), cmp_keyed_desc);
        if (capgap) capgap[rowid] = (nk > cap) ? kw[cap - 1].key - kw[cap].key : INFINITY;
        int64_t keep = nk < cap ? nk : cap;
        int64_t ns = 0;
        for (int a = 0; a < nforced; ++a) sel[ns++] = forced[a];
        for (int64_t a = 0; a < keep; ++a) sel[ns++] = kw[a].j;
        qsort(sel, (size_t)ns, sizeof(int64_t), cmp_i64);
        cnt[rowid] = (int32_t)ns;
        for (int64_t a = 0; a < idx_width; ++a)
          idx[rowid * idx_width + a] = a < ns ? (int32_t)sel[a] : -1;
        if (wsel)
          for (int64_t a = 0; a < idx_width; ++a) {
            double w = 0.0;
            if (a < ns) {
              if (is_forced(sel[a], forced, nforced)) {
                w = 1.0;
              } else {
                for (int64_t k = 0; k < keep; ++k)
                  if (kw[k].j == sel[a]) w = kw[k].key;
              }
            }
            wsel[rowid * idx_width + a] = w;
          }
      }
  free(x);
  free(p);
  free(wbar);
  free(cj);
  free(kw);
  free(sel);
}

/* ------------------------------------------------------------------------- */
/* Stage 2: exact softmax attention over the selected blocks' tokens.         */
/* ------------------------------------------------------------------------- */

/*
 * Fine attention over the tokens of the selected blocks ("DashAttention",
 * Declaração do Problema and Estágio 2 with no routing bias; "SSA", section 2,
 * the block-sparse stream).  Computed only for the requested query rows.
 *
 *   Q : [nb, hq, nq, d];  K, V : [nb, hkv, nk, d]  (fp32).
 *   prefill: nq == nk, query t sits at position t, its routing row is t / B.
 *   token  : as prefill, but query t has a routing row of its own (row t).
 *   decode : nq == 1, query of batch b sits at position kv_lens[b]-1, row 0.
 *   idx/cnt: [nb, hkv, nrow, kmax] / [nb, hkv, nrow] from the router.
 *   req    : [nreq, 3] (b, h, t) query rows to compute (t ignored in decode).
 *   Keys attended: T = union over selected j of block j, restricted to
 *   positions <= the query's position (causal) and < the sequence length.
 *   a_t' = q . k_t' * sm_scale; p = exp(a - max a) / sum; o = sum p v.
 *   An empty T gives o = 0.
 *   wsel  : NULL, or the routing weight w of every listed block (layout of
 *           idx).  Prior-induced softmax ("DashAttention", Estágio 2): the
 *           softmax is taken against a reference g in place of the uniform
 *           one, p maximising z.p - KL(p || g), i.e. p ~ g exp(z); g gives
 *           every token of listed block j the weight w_j^sigma (sigma = 0:
 *           uniform over T, sigma = 1: the routing weights), so the logits
 *           gain sigma * ln w_j.  A listed block with w_j <= 0 has g = 0 and
 *           is left out of T.
 *   O     : [nreq, d] fp64.   pairs : [nreq] (may be NULL) = |T|.
 */
void orc_attend(const float *Q, const float *K, const float *V, int64_t nb, int64_t hq,
                int64_t hkv, int64_t nq, int64_t nk, int64_t d, int64_t B, int mode,
                const int64_t *kv_lens, const int32_t *idx, const int32_t *cnt, int64_t kmax,
                double sm_scale, const int64_t *req, int64_t nreq, double *O, int64_t *pairs,
                const double *wsel, double sigma) {
  (void)nb;
  int64_t G = hq / hkv;
  int64_t nrow = (mode == ORC_MODE_PREFILL) ? (nq + B - 1) / B : (mode == ORC_MODE_TOKEN ? nq : 1);
  int64_t cap = kmax * B + 1;
  double *a = (double *)malloc(sizeof(double) * (size_t)cap);
  double *bias = (double *)malloc(sizeof(double) * (size_t)cap);
  int64_t *tok = (int64_t *)malloc(sizeof(int64_t) * (size_t)cap);
  for (int64_t rq = 0; rq < nreq; ++rq) {
    int64_t b = req[rq * 3 + 0], h = req[rq * 3 + 1], t = req[rq * 3 + 2];
    int64_t g = h / G;
    int64_t pos, row, len;
    if (mode == ORC_MODE_PREFILL || mode == ORC_MODE_TOKEN) {
      pos = t;
      row = mode == ORC_MODE_TOKEN ? t : t / B;
      len = nk;
    } else {
      pos = kv_lens[b] - 1;
      row = 0;
      len = kv_lens[b];
      t = 0;
    }
    const float *qv = Q + ((b * hq + h) * nq + t) * d;
    const float *kb = K + ((b * hkv + g) * nk) * d;
    const float *vb = V + ((b * hkv + g) * nk) * d;
    int64_t rowid = (b * hkv + g) * nrow + row;
    int64_t nt = 0;
    for (int64_t s = 0; s < cnt[rowid]; ++s) {
      int64_t j = idx[rowid * kmax + s];
      double bj = 0.0;
      if (wsel) {
        double w = wsel[rowid * kmax + s];
        if (!(w > 0.0)) continue;
        bj = sigma * log(w);
      }
      for (int64_t tp = j * B; tp < (j + 1) * B && tp < len && tp <= pos; ++tp) {
        bias[nt] = bj;
        tok[nt++] = tp;
      }
    }
    double *o = O + rq * d;
    for (int64_t c = 0; c < d; ++c) o[c] = 0.0;
    if (pairs) pairs[rq] = nt;
    if (nt == 0) continue;
    double mx = -INFINITY;
    for (int64_t u = 0; u < nt; ++u) {
      double acc = 0.0;
      for (int64_t c = 0; c < d; ++c) acc += (double)qv[c] * (double)kb[tok[u] * d + c];
      a[u] = acc * sm_scale + bias[u];
      if (a[u] > mx) mx = a[u];
    }
    double z = 0.0;
    for (int64_t u = 0; u < nt; ++u) {
      a[u] = exp(a[u] - mx);
      z += a[u];
    }
    for (int64_t u = 0; u < nt; ++u) {
      double w = a[u] / z;
      for (int64_t c = 0; c < d; ++c) o[c] += w * (double)vb[tok[u] * d + c];
    }
  }
  free(a);
  free(bias);
  free(tok);
}

/* ------------------------------------------------------------------------- */
/* Stage 2 with per-token selections: the tile's active blocks as a bit mask. */
/* ------------------------------------------------------------------------- */

/*
 * Active-block mask of a query tile ("DashAttention", Estágio 2,
 * Implementação: the attention kernel walks the active blocks given by a
 * bit-packed mask).  Queries are grouped in tiles of 64 consecutive tokens;
 * a block is active for a tile when at least one of its tokens selected it,
 * and bit r of that block's word says whether token 64*tile + r did.
 *
 *   idx/cnt : [nb, hkv, n, width] / [nb, hkv, n] per-token selections
 *             (entries outside [0, nblk) are ignored).
 *   Outputs per (b, g, tile), ntile = ceil(n / 64):
 *     uidx [.., nblk] active blocks in ascending order, -1 padded;
 *     ucnt [..] their number;
 *     ubits[.., nblk] the 64-bit token word of each listed block, 0 padded.
 */
void orc_token_union(const int32_t *idx, const int32_t *cnt, int64_t nb, int64_t hkv, int64_t n,
                     int64_t width, int64_t nblk, int32_t *uidx, int32_t *ucnt, uint64_t *ubits) {
  int64_t ntile = (n + 63) / 64;
  uint64_t *word = (uint64_t *)malloc(sizeof(uint64_t) * (size_t)(nblk > 0 ? nblk : 1));
  for (int64_t b = 0; b < nb; ++b)
    for (int64_t g = 0; g < hkv; ++g)
      for (int64_t tile = 0; tile < ntile; ++tile) {
        for (int64_t j = 0; j < nblk; ++j) word[j] = 0;
        for (int64_t r = 0; r < 64 && tile * 64 + r < n; ++r) {
          int64_t row = (b * hkv + g) * n + tile * 64 + r;
          int64_t c = cnt[row];
          if (c > width) c = width;
          for (int64_t e = 0; e < c; ++e) {
            int64_t j = idx[row * width + e];
            if (j >= 0 && j < nblk) word[j] |= (uint64_t)1 << r;
          }
        }
        int64_t out = ((b * hkv + g) * ntile + tile) * nblk;
        int64_t u = 0;
        for (int64_t j = 0; j < nblk; ++j)
          if (word[j]) {
            uidx[out + u] = (int32_t)j;
            ubits[out + u] = word[j];
            ++u;
          }
        ucnt[(b * hkv + g) * ntile + tile] = (int32_t)u;
        for (int64_t v = u; v < nblk; ++v) {
          uidx[out + v] = -1;
          ubits[out + v] = 0;
        }
      }
  free(word);
}

/* ------------------------------------------------------------------------- */
/* Token-level alpha-entmax attention.                                        */
/* ------------------------------------------------------------------------- */

/*
 * Causal alpha-entmax attention over tokens ("AdaSplash-2", sections 1 and 2:
 * the attention distribution of query t is alpha-entmax of its scores, exact
 * zeros outside a data-dependent support, with the normaliser tau found per
 * query).  For each requested (b, h, t):
 *   x_j = (alpha-1) * sm_scale * q_t . k_j  for keys j <= t (KV head h / G),
 *   tau solves sum_j [x_j - tau]_+^(1/(alpha-1)) = 1, found on the sorted x by
 *   the exact prefix closed forms (alpha 1.5, 2) or 64 bisection steps
 *   (other alpha) of solve_sorted,
 *   p_j = [x_j - tau]_+^(1/(alpha-1)) / (their sum), o = sum_j p_j v_j.
 *   Q : [nb, hq, n, d]; K, V : [nb, hkv, n, d] (fp32).
 *   O : [nreq, d] fp64;  tau_out, support : [nreq] (may be NULL).
 */
void orc_entmax_attend(const float *Q, const float *K, const float *V, int64_t nb, int64_t hq,
                       int64_t hkv, int64_t n, int64_t d, double alpha, double sm_scale,
                       const int64_t *req, int64_t nreq, double *O, double *tau_out,
                       int64_t *support) {
  (void)nb;
  int64_t G = hq / hkv;
  double ex = 1.0 / (alpha - 1.0);
  double *x = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
  double *xs = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
  int64_t *ones = (int64_t *)malloc(sizeof(int64_t) * (size_t)(n > 0 ? n : 1));
  for (int64_t a = 0; a < n; ++a) ones[a] = 1;
  for (int64_t rq = 0; rq < nreq; ++rq) {
    int64_t b = req[rq * 3 + 0], h = req[rq * 3 + 1], t = req[rq * 3 + 2];
    int64_t g = h / G;
    const float *qv = Q + ((b * hq + h) * n + t) * d;
    const float *kb = K + ((b * hkv + g) * n) * d;
    const float *vb = V + ((b * hkv + g) * n) * d;
    int64_t m = t + 1;
    for (int64_t j = 0; j < m; ++j) {
      double acc = 0.0;
      for (int64_t c = 0; c < d; ++c) acc += (double)qv[c] * (double)kb[j * d + c];
      x[j] = (alpha - 1.0) * sm_scale * acc;
      xs[j] = x[j];
    }
    qsort(xs, (size_t)m, sizeof(double), cmp_dbl_desc);
    double tau = solve_sorted(xs, ones, m, alpha);
    double z = 0.0;
    int64_t ns = 0;
    for (int64_t j = 0; j < m; ++j) {
      x[j] = x[j] > tau ? pow(x[j] - tau, ex) : 0.0;
      z += x[j];
      ns += x[j] > 0.0;
    }
    double *o = O + rq * d;
    for (int64_t c = 0; c < d; ++c) o[c] = 0.0;
    for (int64_t j = 0; j < m; ++j) {
      if (x[j] == 0.0) continue;
      double w = x[j] / z;
      for (int64_t c = 0; c < d; ++c) o[c] += w * (double)vb[j * d + c];
    }
    if (tau_out) tau_out[rq] = tau;
    if (support) support[rq] = ns;
  }
  free(x);
  free(xs);
  free(ones);
}

/* ------------------------------------------------------------------------- */
/* Backward of the fine attention over the selected blocks.                   */
/* ------------------------------------------------------------------------- */

/*
 * Gradients of the causal block-sparse attention (Stage 2, prefill rows; the
 * backward pass the pages single out as where training time goes: "SSA",
 * introduction; "AdaSplash-2", section 4, skipping zero blocks) for a fixed
 * selection.  For every query t of head h with attended token set T(t)
 * (as orc_attend, prefill mode):
 *   a_u = sm_scale q_t . k_u, p = softmax(a) over T(t), o_t = sum_u p_u v_u,
 *   D_t = dO_t . o_t,  dp_u = dO_t . v_u,  ds_u = p_u (dp_u - D_t),
 *   dQ_t += sm_scale sum_u ds_u k_u,
 *   dK_u += sm_scale ds_u q_t,  dV_u += p_u dO_t   (KV head h / G: the
 *   group's query heads add into the same dK, dV).
 *   Q, dO : [nb, hq, n, d];  K, V : [nb, hkv, n, d] (fp32); idx/cnt per query
 *   block (mode ORC_MODE_PREFILL) or per query token (ORC_MODE_TOKEN, the
 *   per-token selections of "DashAttention", Estágio 1: row t lists the blocks
 *   query t attends).  dQ [nb, hq, n, d], dK, dV [nb, hkv, n, d]: fp64,
 *   overwritten.
 *   rowmask: NULL, or [nb, hkv, nrow] bytes; then only the queries of the
 *   query blocks whose byte is nonzero contribute (a sample: dQ of those
 *   queries, and dK, dV of every key block all of whose selecting rows are
 *   in it, are exact).
 *   wsel, sigma: the prior-induced softmax of orc_attend (NULL: none); the
 *   logit of a key of listed block j gains sigma ln w_j, entries with
 *   w_j <= 0 are skipped.  dwsel (NULL, or [nb, hkv, nrow, kmax]) receives
 *   dL/dw_j = sigma / w_j * sum of dS over the entry's (query, key) pairs of
 *   every head of the group (0 for skipped entries).
 */
void orc_attend_backward(const float *Q, const float *K, const float *V, const float *dO,
                         int64_t nb, int64_t hq, int64_t hkv, int64_t n, int64_t d, int64_t B,
                         int mode, const int32_t *idx, const int32_t *cnt, int64_t kmax,
                         double sm_scale, const uint8_t *rowmask, const double *wsel,
                         double sigma, double *dwsel, double *dQ, double *dK, double *dV) {
  int64_t G = hq / hkv;
  int64_t rq = mode == ORC_MODE_TOKEN ? 1 : B; /* queries per selection row */
  int64_t nrow = (n + rq - 1) / rq;
  int64_t cap = kmax * B + 1;
  double *p = (double *)malloc(sizeof(double) * (size_t)cap);
  int64_t *tok = (int64_t *)malloc(sizeof(int64_t) * (size_t)cap);
  int64_t *ent = (int64_t *)malloc(sizeof(int64_t) * (size_t)cap);
  double *o = (double *)malloc(sizeof(double) * (size_t)d);
  for (int64_t a = 0; a < nb * hq * n * d; ++a) dQ[a] = 0.0;
  for (int64_t a = 0; a < nb * hkv * n * d; ++a) dK[a] = dV[a] = 0.0;
  if (dwsel)
    for (int64_t a = 0; a < nb * hkv * nrow * kmax; ++a) dwsel[a] = 0.0;
  for (int64_t b = 0; b < nb; ++b)
    for (int64_t h = 0; h < hq; ++h)
      for (int64_t t = 0; t < n; ++t) {
        int64_t g = h / G;
        int64_t rowid = (b * hkv + g) * nrow + t / rq;
        if (rowmask && !rowmask[rowid]) continue;
        const float *qv = Q + ((b * hq + h) * n + t) * d;
        const float *gv = dO + ((b * hq + h) * n + t) * d;
        const float *kb = K + ((b * hkv + g) * n) * d;
        const float *vb = V + ((b * hkv + g) * n) * d;
        double *dq = dQ + ((b * hq + h) * n + t) * d;
        double *dkb = dK + ((b * hkv + g) * n) * d;
        double *dvb = dV + ((b * hkv + g) * n) * d;
        int64_t nt = 0;
        for (int64_t s = 0; s < cnt[rowid]; ++s) {
          int64_t j = idx[rowid * kmax + s];
          if (wsel && !(wsel[rowid * kmax + s] > 0.0)) continue;
          for (int64_t u = j * B; u < (j + 1) * B && u < n && u <= t; ++u) {
            ent[nt] = s;
            tok[nt++] = u;
          }
        }
        if (nt == 0) continue;
        double mx = -INFINITY, z = 0.0;
        for (int64_t a = 0; a < nt; ++a) {
          double acc = 0.0;
          for (int64_t c = 0; c < d; ++c) acc += (double)qv[c] * (double)kb[tok[a] * d + c];
          p[a] = acc * sm_scale;
          if (wsel) p[a] += sigma * log(wsel[rowid * kmax + ent[a]]);
          if (p[a] > mx) mx = p[a];
        }
        for (int64_t a = 0; a < nt; ++a) {
          p[a] = exp(p[a] - mx);
          z += p[a];
        }
        for (int64_t c = 0; c < d; ++c) o[c] = 0.0;
        for (int64_t a = 0; a < nt; ++a) {
          p[a] /= z;
          for (int64_t c = 0; c < d; ++c) o[c] += p[a] * (double)vb[tok[a] * d + c];
        }
        double D = 0.0;
        for (int64_t c = 0; c < d; ++c) D += (double)gv[c] * o[c];
        for (int64_t a = 0; a < nt; ++a) {
          const float *kv = kb + tok[a] * d;
          const float *vv = vb + tok[a] * d;
          double dp = 0.0;
          for (int64_t c = 0; c < d; ++c) dp += (double)gv[c] * (double)vv[c];
          double ds = p[a] * (dp - D);
          if (dwsel) dwsel[rowid * kmax + ent[a]] += ds;
          for (int64_t c = 0; c < d; ++c) {
            dq[c] += sm_scale * ds * (double)kv[c];
            dkb[tok[a] * d + c] += sm_scale * ds * (double)qv[c];
            dvb[tok[a] * d + c] += p[a] * (double)gv[c];
          }
        }
      }
  if (dwsel)
    for (int64_t a = 0; a < nb * hkv * nrow * kmax; ++a)
      dwsel[a] = (wsel && wsel[a] > 0.0) ? dwsel[a] * sigma / wsel[a] : 0.0;
  free(p);
  free(tok);
  free(ent);
  free(o);
}

/* ------------------------------------------------------------------------- */
/* Backward of the entmax routing (the routing weights' gradient reaching the */
/* routing query and the summaries).                                         */
/* ------------------------------------------------------------------------- */

/*
 * Vector-Jacobian product of alpha-entmax written in its logits z
 * (p_j = [(alpha-1) z_j - tau]_+^(1/(alpha-1)), sum p = 1): differentiating
 * the constraint gives dp_j = g_j (dz_j - <g, dz> / sum g) with
 * g_j = p_j^(2-alpha) on the support and 0 off it, so the gradient of a loss
 * with dL/dp = dp is dz_j = g_j (dp_j - <g, dp> / sum g).  ("DashAttention",
 * Estágio 1: entmax routing is differentiable, unlike top-k.)
 */
void orc_entmax_vjp(const double *p, const double *dp, int64_t n, double alpha, double *dz) {
  double sg = 0.0, sgd = 0.0;
  for (int64_t a = 0; a < n; ++a)
    if (p[a] > 0.0) {
      double g = pow(p[a], 2.0 - alpha);
      sg += g;
      sgd += g * dp[a];
    }
  for (int64_t a = 0; a < n; ++a)
    dz[a] = (p[a] > 0.0 && sg > 0.0) ? pow(p[a], 2.0 - alpha) * (dp[a] - sgd / sg) : 0.0;
}

/*
 * Gradient of the loss through the entmax routing of prefill block rows
 * (orc_route_entmax, mode prefill) or of every query token (mode token: the
 * row's routing query is the token's own query and its own block is the
 * diagonal) given dL/dw for the listed blocks
 * (dwsel, layout of idx; from orc_attend_backward).  The listed routed
 * (not forced) block j of row r has w_j = (1/G) sum_h p_hj, so head h's
 * probabilities get dp_hj = dw_j / G (0 for blocks not listed, e.g. cut by
 * the cap); entmax's VJP gives dz over the head's candidates; the logits
 * z_hj = gamma * score_scale * qhat_h . S_j give
 *   dqhat_h += gamma * score_scale * sum_j dz_hj S_j,
 *   dS_j   += gamma * score_scale * sum_{h in group, r} dz_hj qhat_h,
 * and the mean pools (qhat = mean of the row's queries, S = mean of the
 * block's keys, q-bar = 0) spread them evenly: dQ_t = dqhat_row(t) / n_row,
 * dK_u = dS_block(u) / n_block (n = the block's token count; a token row has
 * n_row = 1).
 *   qhat [nb, hq, nrow, d], S [nb, hkv, nblk, d], probs [nb, hq, nrow, nblk]
 *   (fp64, from orc_qpool / orc_summarize / orc_route_entmax);
 *   dQ [nb, hq, n, d], dK [nb, hkv, n, d]: fp64, overwritten with the
 *   routing part only.
 */
void orc_route_entmax_backward(const double *qhat, const double *S, const double *probs,
                               const int32_t *idx, const int32_t *cnt, int64_t idx_width,
                               const double *dwsel, int64_t nb, int64_t hq, int64_t hkv,
                               int64_t n, int64_t d, int64_t B, int mode, double alpha,
                               double gamma, double score_scale, uint32_t force, double *dQ,
                               double *dK) {
  int64_t G = hq / hkv;
  int64_t rq = mode == ORC_MODE_TOKEN ? 1 : B; /* queries pooled per row */
  int64_t nrow = (n + rq - 1) / rq, nblk = (n + B - 1) / B;
  double *dp = (double *)malloc(sizeof(double) * (size_t)nblk);
  double *pc = (double *)malloc(sizeof(double) * (size_t)nblk);
  double *dz = (double *)malloc(sizeof(double) * (size_t)nblk);
  int64_t *cj = (int64_t *)malloc(sizeof(int64_t) * (size_t)nblk);
  double *dqh = (double *)calloc((size_t)(nb * hq * nrow * d), sizeof(double));
  double *dS = (double *)calloc((size_t)(nb * hkv * nblk * d), sizeof(double));
  double f = gamma * score_scale;
  for (int64_t b = 0; b < nb; ++b)
    for (int64_t h = 0; h < hq; ++h)
      for (int64_t r = 0; r < nrow; ++r) {
        int64_t g = h / G;
        int64_t forced[3];
        int nforced = 0;
        int64_t cend = row_setup(mode == ORC_MODE_TOKEN ? ORC_MODE_TOKEN : ORC_MODE_PREFILL, 1, r,
                                 0, B, force, forced, &nforced);
        int64_t rowid = (b * hkv + g) * nrow + r, hrow = (b * hq + h) * nrow + r;
        for (int64_t j = 0; j < nblk; ++j) dp[j] = 0.0;
        for (int64_t a = 0; a < cnt[rowid]; ++a) {
          int64_t j = idx[rowid * idx_width + a];
          if (j >= 0 && j < nblk && !is_forced(j, forced, nforced))
            dp[j] += dwsel[rowid * idx_width + a] / (double)G;
        }
        /* the head's candidates, as routed */
        int64_t nc = 0;
        for (int64_t j = 0; j < cend; ++j)
          if (!is_forced(j, forced, nforced)) cj[nc++] = j;
        double *dpl = (double *)malloc(sizeof(double) * (size_t)(nc + 1));
        for (int64_t a = 0; a < nc; ++a) {
          pc[a] = probs[hrow * nblk + cj[a]];
          dpl[a] = dp[cj[a]];
        }
        orc_entmax_vjp(pc, dpl, nc, alpha, dz);
        free(dpl);
        const double *qv = qhat + hrow * d;
        double *dq = dqh + hrow * d;
        for (int64_t a = 0; a < nc; ++a) {
          if (dz[a] == 0.0) continue;
          const double *sv = S + ((b * hkv + g) * nblk + cj[a]) * d;
          double *ds = dS + ((b * hkv + g) * nblk + cj[a]) * d;
          for (int64_t c = 0; c < d; ++c) {
            dq[c] += f * dz[a] * sv[c];
            ds[c] += f * dz[a] * qv[c];
          }
        }
      }
  for (int64_t b = 0; b < nb; ++b) {
    for (int64_t h = 0; h < hq; ++h)
      for (int64_t t = 0; t < n; ++t) {
        int64_t r = t / rq, nr = (r + 1) * rq < n ? rq : n - r * rq;
        for (int64_t c = 0; c < d; ++c)
          dQ[((b * hq + h) * n + t) * d + c] = dqh[((b * hq + h) * nrow + r) * d + c] / (double)nr;
      }
    for (int64_t g = 0; g < hkv; ++g)
      for (int64_t u = 0; u < n; ++u) {
        int64_t j = u / B, nj = (j + 1) * B < n ? B : n - j * B;
        for (int64_t c = 0; c < d; ++c)
          dK[((b * hkv + g) * n + u) * d + c] = dS[((b * hkv + g) * nblk + j) * d + c] / (double)nj;
      }
  }
  free(dp);
  free(pc);
  free(dz);
  free(cj);
  free(dqh);
  free(dS);
}

/* ------------------------------------------------------------------------- */
/* Backward of the token-level alpha-entmax attention.                        */
/* ------------------------------------------------------------------------- */

/*
 * Gradients of orc_entmax_attend's output for upstream dO ("AdaSplash-2",
 * sections 1 and 4: the entmax attention is trained, its backward skipping
 * the zero blocks).  Per query t of head h: p over the keys j <= t as in the
 * forward (exact tau), dp_j = dO_t . v_j, dz = the entmax VJP of dp
 * (orc_entmax_vjp: g = p^(2-alpha) on the support), and with
 * z_j = sm_scale q_t . k_j:
 *   dQ_t = sm_scale sum_j dz_j k_j,  dK_j += sm_scale dz_j q_t,
 *   dV_j += p_j dO_t   (keys summed over the group's heads).
 *   Q, dO : [nb, hq, n, d];  K, V : [nb, hkv, n, d] (fp32);
 *   dQ, dK, dV fp64, overwritten.
 */
void orc_entmax_attend_backward(const float *Q, const float *K, const float *V, const float *dO,
                                int64_t nb, int64_t hq, int64_t hkv, int64_t n, int64_t d,
                                double alpha, double sm_scale, double *dQ, double *dK,
                                double *dV) {
  int64_t G = hq / hkv;
  double ex = 1.0 / (alpha - 1.0);
  double *x = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
  double *xs = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
  double *dp = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
  double *dz = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
  int64_t *ones = (int64_t *)malloc(sizeof(int64_t) * (size_t)(n > 0 ? n : 1));
  for (int64_t a = 0; a < n; ++a) ones[a] = 1;
  for (int64_t a = 0; a < nb * hq * n * d; ++a) dQ[a] = 0.0;
  for (int64_t a = 0; a < nb * hkv * n * d; ++a) dK[a] = dV[a] = 0.0;
  for (int64_t b = 0; b < nb; ++b)
    for (int64_t h = 0; h < hq; ++h)
      for (int64_t t = 0; t < n; ++t) {
        int64_t g = h / G;
        const float *qv = Q + ((b * hq + h) * n + t) * d;
        const float *gv = dO + ((b * hq + h) * n + t) * d;
        const float *kb = K + ((b * hkv + g) * n) * d;
        const float *vb = V + ((b * hkv + g) * n) * d;
        double *dq = dQ + ((b * hq + h) * n + t) * d;
        double *dkb = dK + ((b * hkv + g) * n) * d;
        double *dvb = dV + ((b * hkv + g) * n) * d;
        int64_t m = t + 1;
        for (int64_t j = 0; j < m; ++j) {
          double acc = 0.0;
          for (int64_t c = 0; c < d; ++c) acc += (double)qv[c] * (double)kb[j * d + c];
          x[j] = (alpha - 1.0) * sm_scale * acc;
          xs[j] = x[j];
        }
        qsort(xs, (size_t)m, sizeof(double), cmp_dbl_desc);
        double tau = solve_sorted(xs, ones, m, alpha);
        double z = 0.0;
        for (int64_t j = 0; j < m; ++j) {
          x[j] = x[j] > tau ? pow(x[j] - tau, ex) : 0.0;
          z += x[j];
        }
        for (int64_t j = 0; j < m; ++j) {
          x[j] /= z; /* p */
          double acc = 0.0;
          for (int64_t c = 0; c < d; ++c) acc += (double)gv[c] * (double)vb[j * d + c];
          dp[j] = acc;
        }
        orc_entmax_vjp(x, dp, m, alpha, dz);
        for (int64_t j = 0; j < m; ++j) {
          if (x[j] == 0.0) continue;
          for (int64_t c = 0; c < d; ++c) {
            dq[c] += sm_scale * dz[j] * (double)kb[j * d + c];
            dkb[j * d + c] += sm_scale * dz[j] * (double)qv[c];
            dvb[j * d + c] += x[j] * (double)gv[c];
          }
        }
      }
  free(x);
  free(xs);
  free(dp);
  free(dz);
  free(ones);
}
