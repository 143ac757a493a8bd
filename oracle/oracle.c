/*
 * oracle.c - plain CPU oracle of the sparsely-gated MoE layer forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header or table with the HIP library, and it never receives a value that
 * the HIP library produced.
 *
 * What it computes (page names are the titles of the source web pages):
 *
 *   y(x) = sum_i G(x)_i * E_i(x),  G(x) = softmax(KeepTopK(x W_g, k))
 *     - "Sparsely-Gated MoE" paper summary (Qiita), sections "Sparsely-Gated
 *       MoE layer formula" and "Gating: Noisy Top-k Softmax" (the
 *       inference-time, noise-free form).
 *   Router scores in float32, one term at a time, then a stable descending
 *   sort (ties keep the lower expert index), the first k kept, and a
 *   softmax over those k only, with the maximum subtracted
 *     - Go book chapter "MoE (Mixture of Experts)", section 2 "Routing:
 *       pick the top k and re-softmax" (Route).
 *   Token loop: count each chosen expert, run its FFN, add weight * output
 *     - same chapter and section (Forward, Stats).
 *   Expert FFN: Linear -> GELU -> Linear (4x wider hidden layer)
 *     - "Extending Raschka's GPT-2: an MoE ..." summary (techfeed), section
 *       "How MoE works: split the FFN"; Go chapter, "What was simplified"
 *       (GELU experts; real ones such as Mixtral use SwiGLU).
 *   SwiGLU expert with gate and up projections packed into one
 *   [E, 2h, d] tensor (rows 0..h-1 gate/w1, rows h..2h-1 up/w3)
 *     - "Understanding MoE in Transformers", section "Weight Loading
 *       Refactor" (MergeModulelist over experts, Concatenate on dim 1).
 *   Load-balance loss N * sum_e f_e^2, 0 when no token was routed
 *     - Go chapter, section 3 "Load balancing".
 *   Importance(X)_i = sum_x G(x)_i, CV(.)^2 of Importance and Load
 *     - Qiita summary, section "Load-balancing losses".
 *   Parameter accounting Total = d*E + E*P_e, Active = d*E + k*P_e
 *     - Go chapter, section 1 "Parameter accounting".
 *
 * Readings where the pages are silent (each is listed with its reason in
 * the design notes of the repository):
 *   - router dot product: fmaf per term, i ascending, starting from +0.0f,
 *     bias (if any) added after the last term, all in float32;
 *   - softmax weights evaluated in double from the float32 scores;
 *   - GELU is the exact x * Phi(x) (erf form);
 *   - expert arithmetic in double from the exact values of the stored
 *     float32 / bfloat16 numbers; no rounding of intermediates;
 *   - Load(X) = hard per-expert counts (no noise at inference);
 *   - CV^2 uses the population variance; 0 when the mean is 0;
 *   - SwiGLU experts count P_e = 3*d*h weights, GELU experts 2*d*h; a
 *     shared always-on expert adds P_e to both totals;
 *   - within an expert's group, rows keep the order of the flat assignment
 *     index t*k + j;
 *   - expert capacity: an expert accepts its first C assignments in that
 *     flat order, the rest are dropped, the surviving weights are not
 *     renormalised (Go chapter, "What was simplified");
 *   - next-choice re-routing of the overflow (Go chapter, "Design
 *     viewpoints", capacity factor): one hop.  The o-th overflowing slot of
 *     a token (slot order) is offered to the token's o-th best expert
 *     outside its top k (score descending, ties to the lower index); each
 *     expert accepts offers in flat order while it has room left after the
 *     first round; an offer that finds no room is dropped.  The slot keeps
 *     its gate value;
 *   - gate modes other than the default (cfg.gate):
 *     bias-selects: the router bias steers the selection only, the kept
 *     weights are the softmax of the unbiased kept scores (Go chapter,
 *     section 3 "Load balancing" and "Pros, cons and real examples":
 *     DeepSeek-V3 balances load by adjusting a bias instead of a loss);
 *     softmax-all: the softmax runs over all E scores and the kept values
 *     are used as they are, not renormalised (techfeed summary, "The
 *     hardest part: making the router trainable": the softmaxed router
 *     output weights the chosen experts; with k = 1 this is the Switch
 *     Transformer top-1 gate).  Selection is the same stable top-k on the
 *     (biased) float32 scores in every mode.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -mfma (no other contraction).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

#define ORACLE_GELU 0
#define ORACLE_SWIGLU 1
#define ORACLE_F32 0
#define ORACLE_BF16 1

#define ORACLE_GATE_TOPK 0
#define ORACLE_GATE_BIAS_SELECTS 1
#define ORACLE_GATE_SOFTMAX_ALL 2

typedef struct {
  int64_t T;
  int32_t d, h, E, k, S, act, dtype, gate;
} oracle_cfg;

typedef struct {
  const float *w_gate; /* [E, d] float32 */
  const float *b_gate; /* [E] float32 or NULL */
  const void *w_up;    /* GELU [E, h, d]; SwiGLU [E, 2h, d] */
  const void *w_down;  /* [E, d, h] */
  const void *b_up;    /* GELU [E, h] or NULL */
  const void *b_down;  /* GELU [E, d] or NULL */
  const void *w_up_shared;   /* [S, 2h, d] or NULL */
  const void *w_down_shared; /* [S, d, h] or NULL */
} oracle_weights;

/* ---- element access: the exact value of a stored float32 / bfloat16 ---- */

static float bf16_value(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16; /* bfloat16 is the top half of a float32 */
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

static float elem_f(const void *base, int dtype, int64_t i) {
  if (dtype == ORACLE_F32) return ((const float *)base)[i];
  return bf16_value(((const uint16_t *)base)[i]);
}

static double elem(const void *base, int dtype, int64_t i) {
  return (double)elem_f(base, dtype, i);
}

static int cfg_ok(const oracle_cfg *c) {
  return c && c->T >= 0 && c->d > 0 && c->h > 0 && c->E > 0 && c->k >= 1 &&
         c->k <= c->E && (c->S == 0 || c->S == 1) &&
         (c->act == ORACLE_GELU || c->act == ORACLE_SWIGLU) &&
         (c->dtype == ORACLE_F32 || c->dtype == ORACLE_BF16) &&
         !(c->S && c->act != ORACLE_SWIGLU) &&
         c->gate >= ORACLE_GATE_TOPK && c->gate <= ORACLE_GATE_SOFTMAX_ALL;
}

/* ---- step 1: router scores of one token (float32, sequential).  score[e]
 * includes the bias; raw[e] is the same chain without it. ---- */

static void router_scores(const oracle_cfg *c, const void *x, const float *wg,
                          const float *bg, int64_t t, float *score, float *raw) {
  const int d = c->d;
  for (int e = 0; e < c->E; ++e) {
    float s = 0.0f;
    for (int i = 0; i < d; ++i)
      s = fmaf(elem_f(x, c->dtype, t * d + i), wg[(int64_t)e * d + i], s);
    raw[e] = s;
    if (bg) s = s + bg[e];
    score[e] = s;
  }
}

/* ---- step 2: KeepTopK as the first k entries of a stable descending sort.
 * A selection sort that only moves on a strictly larger score keeps equal
 * scores in ascending expert order, which is exactly what a stable sort on
 * "greater" does.  IEEE '>' treats +0 and -0 as equal. ---- */

static void keep_top_k(const float *score, int E, int k, int32_t *idx,
                       unsigned char *taken) {
  memset(taken, 0, (size_t)E);
  for (int j = 0; j < k; ++j) {
    int best = -1;
    for (int e = 0; e < E; ++e) {
      if (taken[e]) continue;
      if (best < 0 || score[e] > score[best]) best = e;
    }
    taken[best] = 1;
    idx[j] = best;
  }
}

/* ---- step 3: softmax over the k kept scores (the rest are -inf and get
 * weight exactly 0), maximum subtracted, evaluated in double. ---- */

static void kept_softmax(const float *score, const int32_t *idx, int k,
                         double *w) {
  double m = (double)score[idx[0]];
  for (int j = 1; j < k; ++j)
    if ((double)score[idx[j]] > m) m = (double)score[idx[j]];
  double z = 0.0;
  for (int j = 0; j < k; ++j) {
    w[j] = exp((double)score[idx[j]] - m);
    z += w[j];
  }
  for (int j = 0; j < k; ++j) w[j] = w[j] / z;
}

/* softmax over all E scores, read at the kept indices (no renormalisation
 * over the kept ones). */
static void full_softmax_at(const float *score, int E, const int32_t *idx,
                            int k, double *w) {
  double m = (double)score[0];
  for (int e = 1; e < E; ++e)
    if ((double)score[e] > m) m = (double)score[e];
  double z = 0.0;
  for (int e = 0; e < E; ++e) z += exp((double)score[e] - m);
  for (int j = 0; j < k; ++j) w[j] = exp((double)score[idx[j]] - m) / z;
}

/* The gate values of the kept experts for the configured gate mode. */
static void gate_weights(const oracle_cfg *c, const float *score,
                         const float *raw, const int32_t *idx, double *w) {
  if (c->gate == ORACLE_GATE_BIAS_SELECTS)
    kept_softmax(raw, idx, c->k, w);
  else if (c->gate == ORACLE_GATE_SOFTMAX_ALL)
    full_softmax_at(score, c->E, idx, c->k, w);
  else
    kept_softmax(score, idx, c->k, w);
}

/* ---- step 4: one expert FFN on one token row, in double.
 * e in [0, E) is a routed expert; e == E is the shared expert. ---- */

static double gelu(double a) { return 0.5 * a * (1.0 + erf(a * M_SQRT1_2)); }

static double silu(double g) { return g / (1.0 + exp(-g)); }

static void expert_ffn(const oracle_cfg *c, const oracle_weights *W, int e,
                       const double *xr, double *hid, double *yr) {
  const int64_t d = c->d, h = c->h;
  const int dt = c->dtype;
  const int shared = (e == c->E);
  const void *wu = shared ? W->w_up_shared : W->w_up;
  const void *wd = shared ? W->w_down_shared : W->w_down;
  const int64_t eo = shared ? 0 : e;

  if (c->act == ORACLE_GELU) {
    const int64_t ub = eo * h * d; /* W1[e] is [h, d] */
    for (int64_t n = 0; n < h; ++n) {
      double a = 0.0;
      for (int64_t i = 0; i < d; ++i) a += elem(wu, dt, ub + n * d + i) * xr[i];
      if (W->b_up) a += elem(W->b_up, dt, eo * h + n);
      hid[n] = gelu(a);
    }
  } else {
    const int64_t ub = eo * 2 * h * d; /* [2h, d]: gate rows, then up rows */
    for (int64_t n = 0; n < h; ++n) {
      double g = 0.0, u = 0.0;
      for (int64_t i = 0; i < d; ++i) {
        g += elem(wu, dt, ub + n * d + i) * xr[i];
        u += elem(wu, dt, ub + (h + n) * d + i) * xr[i];
      }
      hid[n] = silu(g) * u;
    }
  }
  const int64_t db = eo * d * h; /* W2[e] is [d, h] */
  for (int64_t o = 0; o < d; ++o) {
    double s = 0.0;
    for (int64_t n = 0; n < h; ++n) s += elem(wd, dt, db + o * h + n) * hid[n];
    if (c->act == ORACLE_GELU && W->b_down) s += elem(W->b_down, dt, eo * d + o);
    yr[o] = s;
  }
}

/* ======================= exported entry points ======================= */

int oracle_max_threads(void) { return omp_get_max_threads(); }
void oracle_set_threads(int n) {
  if (n > 0) omp_set_num_threads(n);
}

/* Routing of tokens t0 .. t0+nt-1: float32 scores (optional), kept expert
 * indices in descending score order, and their double softmax weights. */
int oracle_route(const oracle_cfg *c, const void *x, const float *wg,
                 const float *bg, int64_t t0, int64_t nt, float *scores,
                 int32_t *idx, double *w) {
  if (!cfg_ok(c) || !x || !wg || !idx || !w || t0 < 0 || nt < 0 ||
      t0 + nt > c->T)
    return -1;
  int bad = 0;
#pragma omp parallel reduction(| : bad)
  {
    float *s = (float *)malloc(sizeof(float) * (size_t)c->E);
    float *raw = (float *)malloc(sizeof(float) * (size_t)c->E);
    unsigned char *tk = (unsigned char *)malloc((size_t)c->E);
#pragma omp for schedule(static)
    for (int64_t r = 0; r < nt; ++r) {
      router_scores(c, x, wg, bg, t0 + r, s, raw);
      for (int e = 0; e < c->E; ++e)
        if (!isfinite(s[e]) || !isfinite(raw[e])) bad = 1;
      if (scores) memcpy(scores + r * c->E, s, sizeof(float) * (size_t)c->E);
      keep_top_k(s, c->E, c->k, idx + r * c->k, tk);
      gate_weights(c, s, raw, idx + r * c->k, w + r * c->k);
    }
    free(s);
    free(raw);
    free(tk);
  }
  return bad ? -2 : 0;
}

/* Per-expert counts (Stats.TokensPerExpert) and Importance, token order. */
int oracle_counts(const oracle_cfg *c, const int32_t *idx, const double *w,
                  int32_t *counts, double *importance) {
  if (!cfg_ok(c) || !idx || !counts) return -1;
  for (int e = 0; e < c->E; ++e) {
    counts[e] = 0;
    if (importance) importance[e] = 0.0;
  }
  for (int64_t f = 0; f < c->T * c->k; ++f) {
    const int e = idx[f];
    if (e < 0 || e >= c->E) return -1;
    counts[e] += 1;
    if (importance && w) importance[e] += w[f];
  }
  return 0;
}

/* Grouping of the T*k assignments by expert: offsets[E+1] (exclusive scan of
 * the counts), perm_src[p] = source token of row p, pos[t*k+j] = row of
 * assignment (t, j).  Rows of one expert keep flat-index order. */
int oracle_permute(const oracle_cfg *c, const int32_t *idx, int32_t *offsets,
                   int32_t *perm_src, int32_t *pos) {
  if (!cfg_ok(c) || !idx || !offsets || !perm_src || !pos) return -1;
  const int64_t n = c->T * c->k;
  int64_t p = 0;
  for (int e = 0; e < c->E; ++e) {
    offsets[e] = (int32_t)p;
    for (int64_t f = 0; f < n; ++f) {
      if (idx[f] != e) continue;
      perm_src[p] = (int32_t)(f / c->k);
      pos[f] = (int32_t)p;
      ++p;
    }
  }
  offsets[c->E] = (int32_t)p;
  return p == n ? 0 : -1;
}

/* Expert capacity (Go chapter, "What was simplified": real implementations
 * cap the tokens an expert accepts and drop the overflow).  Reading: expert
 * e accepts its first `capacity` assignments in flat order f = t*k + j
 * (token order, and a token's higher-scored slot first); keep[f] = 1 for
 * those, 0 for the dropped ones.  capacity = 0 means no limit. */
int oracle_capacity_keep(const oracle_cfg *c, const int32_t *idx, int32_t capacity,
                         unsigned char *keep) {
  if (!cfg_ok(c) || !idx || !keep || capacity < 0) return -1;
  int64_t *taken = (int64_t *)calloc((size_t)c->E, sizeof(int64_t));
  for (int64_t f = 0; f < c->T * c->k; ++f) {
    const int e = idx[f];
    if (e < 0 || e >= c->E) {
      free(taken);
      return -1;
    }
    keep[f] = (capacity == 0 || taken[e] < capacity) ? 1 : 0;
    taken[e] += 1;
  }
  free(taken);
  return 0;
}

/* Grouping with a capacity: only kept assignments get rows; offsets[E+1]
 * over the kept rows, perm_src[p] for p < offsets[E], pos[f] = -1 for a
 * dropped assignment. */
int oracle_permute_keep(const oracle_cfg *c, const int32_t *idx,
                        const unsigned char *keep, int32_t *offsets,
                        int32_t *perm_src, int32_t *pos) {
  if (!cfg_ok(c) || !idx || !keep || !offsets || !perm_src || !pos) return -1;
  const int64_t n = c->T * c->k;
  int64_t p = 0;
  for (int64_t f = 0; f < n; ++f) pos[f] = -1;
  for (int e = 0; e < c->E; ++e) {
    offsets[e] = (int32_t)p;
    for (int64_t f = 0; f < n; ++f) {
      if (idx[f] != e || !keep[f]) continue;
      perm_src[p] = (int32_t)(f / c->k);
      pos[f] = (int32_t)p;
      ++p;
    }
  }
  offsets[c->E] = (int32_t)p;
  return 0;
}

/* Next-choice re-routing under a capacity (Go chapter, "Design viewpoints":
 * an overflowing token is dropped or handed to its next candidate).  One hop:
 *   1. expert e accepts its first C assignments in flat order f = t*k + j
 *      (the drop rule above);
 *   2. the o-th overflowing slot of token t (o counted in slot order) is
 *      offered to the o-th best expert among those not in t's top k, best
 *      meaning the higher score, ties to the lower index (no offer if there
 *      are fewer than o + 1 such experts);
 *   3. each expert accepts the offers in flat order while it has fewer than
 *      C assignments; the rest are dropped.
 * scores [T, E] float32 (the router scores the selection was taken on);
 * assign[f] = the expert that computes slot f, or -1 if it is dropped.  The
 * gate value of a slot is not changed by where it is computed. */
static const float *rank_scores;   /* comparator context (single-threaded use) */
static int by_score_then_index(const void *a, const void *b) {
  const int ea = *(const int *)a, eb = *(const int *)b;
  const float sa = rank_scores[ea], sb = rank_scores[eb];
  if (sa > sb) return -1;
  if (sa < sb) return 1;
  return ea < eb ? -1 : (ea > eb);
}

int oracle_capacity_reroute(const oracle_cfg *c, const int32_t *idx, const float *scores,
                            int32_t capacity, int32_t *assign) {
  if (!cfg_ok(c) || !idx || !scores || !assign || capacity < 0) return -1;
  const int64_t n = c->T * c->k;
  const int E = c->E, k = c->k;
  for (int64_t i = 0; i < c->T * E; ++i)
    if (!isfinite(scores[i])) return -2;
  int64_t *taken = (int64_t *)calloc((size_t)E, sizeof(int64_t));
  int *cand = (int *)malloc(sizeof(int) * (size_t)E);
  unsigned char *in_top = (unsigned char *)malloc((size_t)E);
  int rc = 0;
  /* 1. first round: the drop rule; -2 marks an overflowing slot */
  for (int64_t f = 0; f < n && rc == 0; ++f) {
    const int e = idx[f];
    if (e < 0 || e >= E) {
      rc = -1;
      break;
    }
    if (capacity == 0 || taken[e] < capacity) {
      assign[f] = e;
      taken[e] += 1;
    } else {
      assign[f] = -2;
    }
  }
  /* 2. offers: the token's ranked experts outside its top k */
  int32_t *offer = (int32_t *)malloc(sizeof(int32_t) * (size_t)(n > 0 ? n : 1));
  for (int64_t t = 0; t < c->T && rc == 0; ++t) {
    for (int e = 0; e < E; ++e) in_top[e] = 0;
    for (int j = 0; j < k; ++j) in_top[idx[t * k + j]] = 1;
    int nc = 0;
    for (int e = 0; e < E; ++e)
      if (!in_top[e]) cand[nc++] = e;
    rank_scores = scores + t * E;
    qsort(cand, (size_t)nc, sizeof(int), by_score_then_index);
    int o = 0;
    for (int j = 0; j < k; ++j) {
      const int64_t f = t * k + j;
      offer[f] = -1;
      if (assign[f] != -2) continue;
      if (o < nc) offer[f] = cand[o];
      ++o;
    }
  }
  /* 3. second round: offers accepted in flat order while there is room */
  for (int64_t f = 0; f < n && rc == 0; ++f) {
    if (assign[f] != -2) continue;
    const int e = offer[f];
    if (e >= 0 && taken[e] < capacity) {
      assign[f] = e;
      taken[e] += 1;
    } else {
      assign[f] = -1;
    }
  }
  free(offer);
  free(taken);
  free(cand);
  free(in_top);
  return rc;
}

/* Grouping by the computing expert of each slot (assign[f], -1 = dropped):
 * offsets[E+1] over the computed rows, perm_src[p] for p < offsets[E],
 * pos[f] = -1 for a dropped slot; rows in flat order within a group. */
int oracle_permute_assign(const oracle_cfg *c, const int32_t *assign, int32_t *offsets,
                          int32_t *perm_src, int32_t *pos) {
  if (!cfg_ok(c) || !assign || !offsets || !perm_src || !pos) return -1;
  const int64_t n = c->T * c->k;
  for (int64_t f = 0; f < n; ++f)
    if (assign[f] < -1 || assign[f] >= c->E) return -1;
  int64_t p = 0;
  for (int64_t f = 0; f < n; ++f) pos[f] = -1;
  for (int e = 0; e < c->E; ++e) {
    offsets[e] = (int32_t)p;
    for (int64_t f = 0; f < n; ++f) {
      if (assign[f] != e) continue;
      perm_src[p] = (int32_t)(f / c->k);
      pos[f] = (int32_t)p;
      ++p;
    }
  }
  offsets[c->E] = (int32_t)p;
  return 0;
}

/* One expert (e < E routed, e == E shared) applied to one row, in double. */
int oracle_expert(const oracle_cfg *c, const oracle_weights *W, int e,
                  const double *xr, double *yr) {
  if (!cfg_ok(c) || !W || !xr || !yr || e < 0 || e > c->E) return -1;
  if (e == c->E && !c->S) return -1;
  double *hid = (double *)malloc(sizeof(double) * (size_t)c->h);
  expert_ffn(c, W, e, xr, hid, yr);
  free(hid);
  return 0;
}

/* The expert output of every slot of the listed tokens, before the gate
 * weight: yslot[r][j] = E_{experts[t*k+j]}(x_t) for t = tokens[r], in double
 * (a slot whose expert is -1, a dropped one, gets zeros).  This is the
 * term E_i(x) of y = sum_i G(x)_i E_i(x) for each kept i ("Sparsely-Gated
 * MoE" summary, "Sparsely-Gated MoE layer formula"), one row per slot, so
 * that a test can form the router's share of the gradient, which needs
 * every slot's expert output.  OpenMP over (token, slot) pairs. */
int oracle_slot_outputs(const oracle_cfg *c, const oracle_weights *W, const void *x,
                        const int64_t *tokens, int64_t nt, const int32_t *experts,
                        double *yslot) {
  if (!cfg_ok(c) || !W || !x || !tokens || !experts || !yslot || nt < 0) return -1;
  for (int64_t r = 0; r < nt; ++r)
    if (tokens[r] < 0 || tokens[r] >= c->T) return -1;
  for (int64_t f = 0; f < c->T * c->k; ++f)
    if (experts[f] < -1 || experts[f] >= c->E) return -1;
  const int64_t d = c->d, k = c->k;
#pragma omp parallel
  {
    double *xr = (double *)malloc(sizeof(double) * (size_t)d);
    double *hid = (double *)malloc(sizeof(double) * (size_t)c->h);
#pragma omp for schedule(dynamic, 1)
    for (int64_t q = 0; q < nt * k; ++q) {
      const int64_t t = tokens[q / k];
      const int e = experts[t * k + q % k];
      double *yo = yslot + q * d;
      if (e < 0) {
        for (int64_t i = 0; i < d; ++i) yo[i] = 0.0;
        continue;
      }
      for (int64_t i = 0; i < d; ++i) xr[i] = elem(x, c->dtype, t * d + i);
      expert_ffn(c, W, e, xr, hid, yo);
    }
    free(xr);
    free(hid);
  }
  return 0;
}

/* The whole layer on the listed tokens (the two entry points below). */
static int forward_tokens_impl(const oracle_cfg *c, const oracle_weights *W,
                               const void *x, const int64_t *tokens, int64_t nt,
                               const unsigned char *keep, const int32_t *assign,
                               double *y, int32_t *idx, double *w) {
  if (!cfg_ok(c) || !W || !W->w_gate || !x || !tokens || !y || !idx || !w ||
      nt < 0)
    return -1;
  if (assign)
    for (int64_t f = 0; f < c->T * c->k; ++f)
      if (assign[f] < -1 || assign[f] >= c->E) return -1;
  if (c->S && (!W->w_up_shared || !W->w_down_shared)) return -1;
  for (int64_t r = 0; r < nt; ++r)
    if (tokens[r] < 0 || tokens[r] >= c->T) return -1;
  const int64_t d = c->d;
  int bad = 0;
#pragma omp parallel reduction(| : bad)
  {
    float *s = (float *)malloc(sizeof(float) * (size_t)c->E);
    float *raw = (float *)malloc(sizeof(float) * (size_t)c->E);
    unsigned char *tk = (unsigned char *)malloc((size_t)c->E);
    double *xr = (double *)malloc(sizeof(double) * (size_t)d);
    double *ye = (double *)malloc(sizeof(double) * (size_t)d);
    double *hid = (double *)malloc(sizeof(double) * (size_t)c->h);
#pragma omp for schedule(dynamic, 1)
    for (int64_t r = 0; r < nt; ++r) {
      const int64_t t = tokens[r];
      router_scores(c, x, W->w_gate, W->b_gate, t, s, raw);
      for (int e = 0; e < c->E; ++e)
        if (!isfinite(s[e]) || !isfinite(raw[e])) bad = 1;
      int32_t *ix = idx + r * c->k;
      double *wr = w + r * c->k;
      keep_top_k(s, c->E, c->k, ix, tk);
      gate_weights(c, s, raw, ix, wr);
      for (int64_t i = 0; i < d; ++i) xr[i] = elem(x, c->dtype, t * d + i);
      double *yo = y + r * d;
      for (int64_t i = 0; i < d; ++i) yo[i] = 0.0;
      for (int j = 0; j < c->k; ++j) {
        if (keep && !keep[t * c->k + j]) continue;
        const int e = assign ? assign[t * c->k + j] : ix[j];   /* computing expert */
        if (e < 0) continue;                                   /* dropped */
        expert_ffn(c, W, e, xr, hid, ye);
        for (int64_t i = 0; i < d; ++i) yo[i] += wr[j] * ye[i];
      }
      if (c->S) {
        expert_ffn(c, W, c->E, xr, hid, ye);
        for (int64_t i = 0; i < d; ++i) yo[i] += ye[i];
      }
    }
    free(s);
    free(raw);
    free(tk);
    free(xr);
    free(ye);
    free(hid);
  }
  return bad ? -2 : 0;
}

/* The whole layer on the listed tokens: y[r] = sum_j w_j * E_{idx_j}(x_t)
 * (+ the shared expert with weight 1), accumulated in slot order.  keep
 * (T*k flags from oracle_capacity_keep, or NULL = keep all): a dropped slot
 * adds nothing and the other weights are not renormalised. */
int oracle_forward_tokens_keep(const oracle_cfg *c, const oracle_weights *W,
                               const void *x, const int64_t *tokens, int64_t nt,
                               const unsigned char *keep, double *y, int32_t *idx,
                               double *w) {
  return forward_tokens_impl(c, W, x, tokens, nt, keep, NULL, y, idx, w);
}

/* The same with the computing expert of every slot given (T*k entries from
 * oracle_capacity_reroute, -1 = dropped): y[r] = sum_j w_j *
 * E_{assign_j}(x_t), the gate values w_j those of the top-k selection. */
int oracle_forward_tokens_assign(const oracle_cfg *c, const oracle_weights *W,
                                 const void *x, const int64_t *tokens, int64_t nt,
                                 const int32_t *assign, double *y, int32_t *idx,
                                 double *w) {
  if (!assign) return -1;
  return forward_tokens_impl(c, W, x, tokens, nt, NULL, assign, y, idx, w);
}

/* Side statistics: out[0] = CV^2(Importance), out[1] = CV^2(Load = counts),
 * out[2] = load-balance loss E * sum_e (counts_e / total)^2 (0 if total 0). */
static double cv2(const double *v, int n) {
  double mean = 0.0;
  for (int i = 0; i < n; ++i) mean += v[i];
  mean /= n;
  if (mean == 0.0) return 0.0;
  double var = 0.0;
  for (int i = 0; i < n; ++i) var += (v[i] - mean) * (v[i] - mean);
  var /= n;
  return var / (mean * mean);
}

int oracle_load_stats(const int32_t *counts, const double *importance, int E,
                      double *out) {
  if (!counts || !out || E <= 0) return -1;
  double *v = (double *)malloc(sizeof(double) * (size_t)E);
  double total = 0.0;
  for (int e = 0; e < E; ++e) {
    v[e] = (double)counts[e];
    total += v[e];
  }
  out[0] = importance ? cv2(importance, E) : 0.0;
  out[1] = cv2(v, E);
  double lb = 0.0;
  if (total != 0.0) {
    for (int e = 0; e < E; ++e) lb += (v[e] / total) * (v[e] / total);
    lb *= E;
  }
  out[2] = lb;
  free(v);
  return 0;
}

/* CV^2 (population variance over the squared mean, 0 when the mean is 0) of
 * any per-expert vector, e.g. the smooth Load(X). */
int oracle_cv2(const double *v, int n, double *out) {
  if (!v || !out || n <= 0) return -1;
  *out = cv2(v, n);
  return 0;
}

/* Parameter accounting: router d*E plus per-expert P_e weights (biases are
 * not counted); the shared expert, if any, is always active. */
int oracle_param_counts(const oracle_cfg *c, int64_t *total, int64_t *active) {
  if (!cfg_ok(c) || !total || !active) return -1;
  const int64_t pe = (int64_t)(c->act == ORACLE_GELU ? 2 : 3) * c->d * c->h;
  const int64_t router = (int64_t)c->d * c->E;
  *total = router + (int64_t)c->E * pe + (int64_t)c->S * pe;
  *active = router + (int64_t)c->k * pe + (int64_t)c->S * pe;
  return 0;
}

/* Without a capacity: every slot kept. */
int oracle_forward_tokens(const oracle_cfg *c, const oracle_weights *W,
                          const void *x, const int64_t *tokens, int64_t nt,
                          double *y, int32_t *idx, double *w) {
  return oracle_forward_tokens_keep(c, W, x, tokens, nt, NULL, y, idx, w);
}

/* ---- noisy top-k gating, the training-time form of the Qiita summary's
 * "Gating: Noisy Top-k Softmax":
 *   H_i = (x W_g)_i (+ b_i) + n_i * Softplus((x W_noise)_i),
 *   G = softmax(KeepTopK(H, k)),
 * with n_i ~ N(0, 1) given as input (the caller draws it).  Softplus is
 * evaluated in double from the float32 noise score and rounded to float32;
 * H is one float32 fused multiply-add, so the top-k decision is taken in
 * float32 as for the clean scores.
 *
 * Smooth load (the Qiita summary's "Load-balancing losses" names Load(X) as
 * a smooth estimate of the per-expert sample count; the estimator is that
 * of Shazeer et al. 2017, appendix A): P(x, i) is the probability that
 * expert i stays in the top k when only its own noise is drawn again,
 *   P(x, i) = Phi(((x W_g)_i - kth_excluding(H, k, i)) / Softplus(...)_i),
 * where kth_excluding is the k-th largest entry of H without entry i, and
 * Load(X)_i = sum_x P(x, i).  With k = E every expert always stays: P = 1.
 * A zero noise scale makes P the indicator of clean score > threshold. ---- */

static double softplus_d(double v) {
  return v > 0.0 ? v + log1p(exp(-v)) : log1p(exp(v));
}

static double normal_cdf(double z) { return 0.5 * erfc(-z * M_SQRT1_2); }

/* Tokens t0 .. t0+nt-1.  Outputs (all [nt, ...]): clean float32 scores
 * [E], noise scale Softplus(x W_noise) float32 [E], H float32 [E], kept
 * indices [k] (stable descending order of H), their softmax weights over the
 * kept H in double [k], and P(x, i) in double [E]. */
int oracle_route_noisy(const oracle_cfg *c, const void *x, const float *wg,
                       const float *bg, const float *wn, const float *noise,
                       int64_t t0, int64_t nt, float *clean, float *scale,
                       float *h, int32_t *idx, double *w, double *p) {
  if (!cfg_ok(c) || !x || !wg || !wn || !noise || !clean || !scale || !h ||
      !idx || !w || !p || t0 < 0 || nt < 0 || t0 + nt > c->T)
    return -1;
  if (c->gate != ORACLE_GATE_TOPK) return -1;
  const int E = c->E, k = c->k;
  int bad = 0;
#pragma omp parallel reduction(| : bad)
  {
    float *raw = (float *)malloc(sizeof(float) * (size_t)E);
    float *nr = (float *)malloc(sizeof(float) * (size_t)E);
    float *nraw = (float *)malloc(sizeof(float) * (size_t)E);
    unsigned char *tk = (unsigned char *)malloc((size_t)E);
    int32_t *order = (int32_t *)malloc(sizeof(int32_t) * (size_t)E);
#pragma omp for schedule(static)
    for (int64_t r = 0; r < nt; ++r) {
      const int64_t t = t0 + r;
      float *cs = clean + r * E, *sc = scale + r * E, *hs = h + r * E;
      router_scores(c, x, wg, bg, t, cs, raw);
      router_scores(c, x, wn, NULL, t, nr, nraw);
      for (int e = 0; e < E; ++e) {
        sc[e] = (float)softplus_d((double)nr[e]);
        hs[e] = fmaf(noise[t * E + e], sc[e], cs[e]);
        if (!isfinite(cs[e]) || !isfinite(hs[e])) bad = 1;
      }
      /* the full stable descending order of H; the first k are kept */
      keep_top_k(hs, E, E, order, tk);
      memcpy(idx + r * k, order, sizeof(int32_t) * (size_t)k);
      kept_softmax(hs, idx + r * k, k, w + r * k);
      for (int e = 0; e < E; ++e) tk[e] = 0;
      for (int j = 0; j < k; ++j) tk[order[j]] = 1;
      double *pr = p + r * E;
      for (int e = 0; e < E; ++e) {
        if (k == E) {
          pr[e] = 1.0;
          continue;
        }
        /* k-th largest of H without entry e */
        const double thr = (double)hs[order[tk[e] ? k : k - 1]];
        const double diff = (double)cs[e] - thr;
        if (sc[e] == 0.0f)
          pr[e] = diff > 0.0 ? 1.0 : 0.0;
        else
          pr[e] = normal_cdf(diff / (double)sc[e]);
      }
    }
    free(raw);
    free(nr);
    free(nraw);
    free(tk);
    free(order);
  }
  return bad ? -2 : 0;
}
