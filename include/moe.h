/*
 * moe.h - C ABI of the MI355X (gfx950) sparsely-gated MoE layer forward.
 *
 * The layer computes y = sum_i G(x)_i * E_i(x) with
 * G(x) = softmax(KeepTopK(x W_g, k)): a linear router, the k largest scores
 * kept (ties to the lower expert index), a softmax over those k only, the k
 * selected expert FFNs, and their gate-weighted sum ("Sparsely-Gated MoE"
 * paper summary on Qiita, sections "Sparsely-Gated MoE layer formula" and
 * "Gating: Noisy Top-k Softmax", inference form without noise).  The
 * dispatch -> compute -> collect split of the calls below follows the
 * "Expert Backend" section of "Understanding MoE in Transformers"; the
 * per-token loop it replaces is Route/Forward in section 2 "Routing" of the
 * Go book chapter "MoE (Mixture of Experts)".
 *
 * Conventions shared by every call:
 *  - Device buffers are plain device pointers, dense row-major, 16-byte
 *    aligned, owned by the caller.  The library allocates no device memory
 *    and keeps no state between calls; scratch space comes from a caller
 *    workspace of at least moe_workspace_bytes() bytes.
 *  - Each call validates its arguments on the host, then only enqueues
 *    kernels on `stream`; it never synchronises or reads device memory, so
 *    the calls can be captured in a HIP graph.  On any error status nothing
 *    has been enqueued, except MOE_ERR_HIP (a launch failed).
 *  - T = num_tokens may be 0: counts, importance and stats are then zeroed
 *    and no other buffer is touched.
 *  - dtype (x, expert weights, hidden rows, y) is bf16 or fp32; the router
 *    weights W_g and b_g are always fp32 and the router scores are fp32.
 *  - Results are deterministic: no floating-point atomics anywhere.
 *  - Non-finite inputs give undefined (but memory-safe) results.
 *
 * Sizes: 1 <= E <= 256, 1 <= k <= E, S (shared always-on experts) is 0 or 1
 * and needs SwiGLU, d and h are multiples of 64, T*k + S*T < 2^31.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 10

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARGUMENT = 1,    /* NULL/misaligned pointer, k > E, ... */
  MOE_ERR_UNSUPPORTED = 2,         /* valid but outside the sizes above */
  MOE_ERR_WORKSPACE_TOO_SMALL = 3,
  MOE_ERR_HIP = 4                  /* a kernel launch failed */
} moe_status_t;

typedef enum { MOE_DTYPE_F32 = 0, MOE_DTYPE_BF16 = 1 } moe_dtype_t;

/* Expert FFN.  GELU: Linear(d->h) + bias -> exact GELU (x*Phi(x)) ->
 * Linear(h->d) + bias, the GPT-2 style expert of the techfeed summary
 * ("How MoE works: split the FFN") and the Go chapter.  SwiGLU: silu(x W1^T)
 * * (x W3^T) -> W2, no biases, the Mixtral-style expert the Go chapter's
 * "What was simplified" names. */
typedef enum { MOE_ACT_GELU = 0, MOE_ACT_SWIGLU = 1 } moe_act_t;

/* How the kept gate values come from the router scores s = x W_g^T + b.
 * The selection is the same in every mode: the stable top-k of s.
 *   MOE_GATE_TOPK_SOFTMAX: softmax over the k kept s (Go chapter section 2,
 *     Route: pick the top k and re-softmax).
 *   MOE_GATE_BIAS_SELECTS: the bias steers the selection only; the weights
 *     are the softmax over the kept experts of the unbiased scores x W_g^T
 *     (Go chapter, section 3 and "Pros, cons and real examples": DeepSeek-V3
 *     balances expert load by adjusting a bias rather than with a loss).
 *   MOE_GATE_SOFTMAX_ALL: softmax over all E scores, read at the kept
 *     experts and not renormalised (techfeed summary, "The hardest part:
 *     making the router trainable": the softmaxed router output weights the
 *     chosen experts; with k = 1 this is the Switch Transformer gate). */
typedef enum {
  MOE_GATE_TOPK_SOFTMAX = 0,
  MOE_GATE_BIAS_SELECTS = 1,
  MOE_GATE_SOFTMAX_ALL = 2
} moe_gate_t;

/* What happens to an assignment beyond an expert's capacity.
 *   MOE_OVERFLOW_DROP: it is dropped (see moe_config_t.capacity).
 *   MOE_OVERFLOW_NEXT_CHOICE: it is handed on once (Go chapter, "Design
 *     viewpoints": an overflowing token is dropped or passed to its next
 *     candidate).  After the first round (the drop rule), the o-th
 *     overflowing slot of a token (slot order) is offered to the token's
 *     o-th best expert outside its top k (higher score first, ties to the
 *     lower index); every expert accepts offers in flat order t*k + j while
 *     it holds fewer than C assignments; an offer that finds no room is
 *     dropped.  A re-routed slot keeps its gate value (the router's output
 *     for that slot) and is computed by the expert it was handed to. */
typedef enum { MOE_OVERFLOW_DROP = 0, MOE_OVERFLOW_NEXT_CHOICE = 1 } moe_overflow_t;

typedef struct {
  int64_t num_tokens;  /* T */
  int32_t d_model;     /* d */
  int32_t d_hidden;    /* h */
  int32_t num_experts; /* E, routed experts */
  int32_t top_k;       /* k */
  int32_t num_shared;  /* S, 0 or 1: always-on expert with weight 1 */
  int32_t act;         /* moe_act_t */
  int32_t dtype;       /* moe_dtype_t */
  int32_t capacity;    /* expert capacity C: 0 = no limit; C >= 1: each expert
                          accepts its first C assignments in flat order
                          t*k + j (token order, then slot order) and the rest
                          are dropped: they add nothing to y and the other
                          weights are not renormalised (the Go chapter's
                          "What was simplified": real implementations cap
                          what an expert accepts and drop the overflow).
                          See moe_expert_capacity for C from a factor. */
  int32_t gate;        /* moe_gate_t (0 = softmax over the kept k) */
  int32_t overflow;    /* moe_overflow_t (0 = drop); used when capacity > 0 */
} moe_config_t;

/* Storage order of the expert matrices (w_up, w_down, w_up_shared,
 * w_down_shared); the router and the biases are always row-major. */
typedef enum {
  MOE_LAYOUT_ROW_MAJOR = 0, /* [rows, cols], cols contiguous */
  MOE_LAYOUT_TILED = 1      /* bf16 only: the blocked order of moe_tile_weights,
                               which the expert GEMMs load as whole 1 KB blocks */
} moe_layout_t;

/* Expert weights, all packed over experts into single tensors ("Weight
 * Loading Refactor" section of "Understanding MoE in Transformers").
 * Every matrix is [out_features, in_features] with in_features contiguous
 * (layout MOE_LAYOUT_ROW_MAJOR, the zero value), or the same numbers in the
 * tiled order (MOE_LAYOUT_TILED; forward calls only: moe_backward returns
 * MOE_ERR_UNSUPPORTED for it, and so does any call of an fp32 layer). */
typedef struct {
  const float *w_gate;   /* router W_g [E, d] fp32 (required) */
  const float *b_gate;   /* router bias [E] fp32, or NULL (added to the score) */
  const void *w_up;      /* GELU: W1 [E, h, d]; SwiGLU: [E, 2h, d] with rows
                            0..h-1 the gate (w1) and rows h..2h-1 the up (w3) */
  const void *b_up;      /* GELU only: [E, h] or NULL; must be NULL for SwiGLU */
  const void *w_down;    /* W2 [E, d, h] */
  const void *b_down;    /* GELU only: [E, d] or NULL; must be NULL for SwiGLU */
  const void *w_up_shared;   /* S = 1: [1, 2h, d], else NULL */
  const void *w_down_shared; /* S = 1: [1, d, h], else NULL */
  int32_t layout;            /* moe_layout_t of the four expert matrices */
} moe_weights_t;

int moe_abi_version(void);
const char *moe_status_string(moe_status_t status);

/* Workspace bytes needed by moe_forward (also enough for moe_permute,
 * moe_expert_ffn and moe_route_noisy).  Pure host; *bytes is 0 when T == 0. */
moe_status_t moe_workspace_bytes(const moe_config_t *cfg, size_t *bytes);

/* Rows of the grouped (expert-sorted) buffers: R = T*k + S*T.  Rows
 * [0, T*k) hold the routed assignments grouped by expert; rows
 * [T*k, T*k + T) hold the shared expert's rows in token order. */
moe_status_t moe_grouped_rows(const moe_config_t *cfg, int64_t *rows);

/* Router + KeepTopK + softmax over the kept scores (Go chapter section 2,
 * Route; Qiita summary, "Gating: Noisy Top-k Softmax", inference form).
 *   x        [T, d] dtype            (device, in)
 *   w_gate   [E, d] fp32, b_gate [E] fp32 or NULL (device, in)
 *   topk_idx [T, k] int32  (out) expert indices in descending score order;
 *            equal scores keep the lower index first (a stable sort)
 *   topk_w   [T, k] fp32   (out) the gate values of cfg->gate; default
 *            exp(s_j - s_0) / sum_i exp(s_i - s_0) over the kept i
 *   counts   [E] int32 or NULL (out) tokens routed to each expert (Stats);
 *            NULL skips them (moe_permute can count them instead)
 *   logits   [T, E] fp32 or NULL (out) router scores: for each (t, e)
 *            s = +0; s = fma(x[t,i], W_g[e,i], s) for i = 0..d-1 in order;
 *            s = s + b_g[e]; all in fp32 (the biased score, in every
 *            gate mode) */
moe_status_t moe_route(const moe_config_t *cfg, const void *x,
                       const float *w_gate, const float *b_gate,
                       int32_t *topk_idx, float *topk_w, int32_t *counts,
                       float *logits, hipStream_t stream);

/* Noisy top-k gating, the training-time gate of the Qiita summary ("Gating:
 * Noisy Top-k Softmax"): H_i = s_i + n_i * Softplus((x W_noise)_i), where s
 * is the router score of moe_route (bias included) and n ~ N(0, 1) is drawn
 * by the caller; G = softmax(KeepTopK(H, k)).  Softplus is evaluated in
 * double from the fp32 noise score and rounded to fp32; H is one fp32 fused
 * multiply-add.  Also the smooth Load of the same summary ("Load-balancing
 * losses": a smooth estimate of each expert's sample count), with the
 * estimator of Shazeer et al.: P(x, i) = Phi((s_i - t_i) / Softplus_i), t_i
 * the k-th largest H without entry i (P = 1 when k = E; a zero scale gives
 * the indicator of s_i > t_i); Load_i = sum over tokens of P(x, i).
 * cfg->gate must be MOE_GATE_TOPK_SOFTMAX (else MOE_ERR_UNSUPPORTED).
 *   x, w_gate, b_gate   as for moe_route     (device, in)
 *   w_noise      [E, d] fp32                 (device, in)
 *   noise        [T, E] fp32 N(0,1) draws    (device, in)
 *   clean_logits [T, E] fp32 (out) s, the moe_route scores
 *   noise_scale  [T, E] fp32 (out) Softplus(x W_noise^T)
 *   topk_idx, topk_w [T, k] (out) kept experts in descending H order (ties
 *                to the lower index) and their softmax over the kept H
 *   counts [E] int32 (out); importance [E] fp32 (out) sum of the kept
 *                weights; load [E] fp32 (out) the smooth Load
 *   cv2    [2] fp64 or NULL (out) CV^2(Importance), CV^2(Load)
 *   workspace    >= moe_workspace_bytes(cfg) bytes (device, scratch)
 * Sums are taken in a fixed order: results are deterministic. */
moe_status_t moe_route_noisy(const moe_config_t *cfg, const void *x,
                             const float *w_gate, const float *b_gate,
                             const float *w_noise, const float *noise,
                             float *clean_logits, float *noise_scale,
                             int32_t *topk_idx, float *topk_w, int32_t *counts,
                             float *importance, float *load, double *cv2,
                             void *workspace, size_t workspace_bytes,
                             hipStream_t stream);

/* Dispatch: stable grouping of the T*k assignments by expert (ties by the
 * flat index t*k + j) and the row move x -> x_perm ("Expert Backend":
 * sort and group tokens by expert id before the grouped GEMM).
 *   topk_idx, topk_w [T, k]   (device, in) as written by moe_route
 *   logits     [T, E] fp32    (device, in) moe_route's scores; read only
 *              under a capacity with MOE_OVERFLOW_NEXT_CHOICE (the next
 *              choices are ranked by them), else ignored (may be NULL).
 *              Re-routing is defined for moe_route's selection only: the
 *              noisy gate selects on H, which no call outputs, so a
 *              selection of moe_route_noisy is not to be re-routed
 *   x          [T, d] dtype   (device, in)
 *   offsets    [E + 1] int32  (out) group starts of the kept assignments;
 *              offsets[E] = T*k without a capacity, else the number of
 *              computed assignments (sum_e min(n_e, C) under the drop rule)
 *   perm_src   [T*k] int32    (out) source token of grouped row p, for
 *              p < offsets[E]
 *   pos        [T*k] int32    (out) grouped row of assignment (t, j), or -1
 *              if the expert capacity dropped it; under next-choice
 *              re-routing the row lies in the group of the expert that
 *              computes the slot (rows in flat order within a group)
 *   importance [E] fp32       (out) Importance(X)_e = sum of the router
 *              weights routed to e (Qiita summary, "Load-balancing losses"),
 *              fp32, in a fixed order (64 lane-strided partial sums over
 *              the group's rows, then a fixed butterfly), so deterministic;
 *              dropped assignments included (they are the router's output)
 *   stats      [3] double or NULL (out) CV^2(Importance), CV^2(Load) with
 *              Load = counts, and the load-balance loss E*sum_e f_e^2 of the
 *              Go chapter's section 3 (population variance; 0 if empty)
 *   counts     [E] int32 or NULL (out) assignments per expert (every one,
 *              dropped or not: moe_route's counts), from the grouping's
 *              histogram
 *   x_perm     [T*k, d] dtype (out) x_perm[p] = x[perm_src[p]] for
 *              p < offsets[E]; or NULL: no rows are moved (the grouping
 *              only; moe_expert_up can read the rows of x in place)
 *   ws         workspace >= moe_workspace_bytes() */
moe_status_t moe_permute(const moe_config_t *cfg, const int32_t *topk_idx,
                         const float *topk_w, const float *logits, const void *x,
                         int32_t *offsets,
                         int32_t *perm_src, int32_t *pos, float *importance,
                         double *stats, int32_t *counts, void *x_perm, void *ws,
                         size_t ws_bytes, hipStream_t stream);

/* moe_permute without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  The scratch is a static device array
 * of MOE_NOALLOC_SCRATCH_BYTES per GPU inside the library (its address is
 * looked up once per device, on the first call there; the array lives until
 * the process ends).  Arguments and results as for moe_permute.  A
 * configuration whose dispatch scratch exceeds the array (T*k beyond about
 * 2^21 assignments with next-choice re-routing, more without) returns
 * MOE_ERR_WORKSPACE_TOO_SMALL before anything is enqueued.  Every call on a
 * GPU shares that GPU's array: calls that overlap on one GPU (other streams,
 * other host threads) race and give undefined results; calls in one stream
 * are ordered and safe.  No call leaves state that a later one relies on. */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)
moe_status_t moe_permute_noalloc(const moe_config_t *cfg, const int32_t *topk_idx,
                                 const float *topk_w, const float *logits, const void *x,
                                 int32_t *offsets, int32_t *perm_src, int32_t *pos,
                                 float *importance, double *stats, int32_t *counts,
                                 void *x_perm, hipStream_t stream);

/* Up projection + activation of every expert group (grouped GEMM on bf16
 * MFMA, fp32 accumulation; fp32 SIMT for dtype fp32).  Experts with no rows
 * are skipped (conditional computation: Qiita summary, "Sparsely-Gated MoE
 * layer formula").
 *   The token rows of the routed groups come from x_perm [T*k, d] (grouped
 *   by moe_permute), or, when x_perm is NULL, straight from x: grouped row
 *   p is x[perm_src[p]] (perm_src [T*k] int32 from moe_permute), so the
 *   grouped copy is never written.  The gathered form needs T*d*bytes <
 *   2^31 (else MOE_ERR_UNSUPPORTED).
 *   x [T, d] (the shared expert's input, and the gathered rows' source; may
 *   be NULL if S = 0 and x_perm is given); perm_src ignored if x_perm given
 *   offsets [E + 1] int32
 *   hidden [R, h] dtype (out) activation rows, R = T*k + S*T */
moe_status_t moe_expert_up(const moe_config_t *cfg, const moe_weights_t *w,
                           const void *x_perm, const int32_t *perm_src,
                           const void *x, const int32_t *offsets, void *hidden,
                           hipStream_t stream);

/* The up projection of a training step: moe_expert_up, and the expert
 * pre-activations that the backward pass differentiates through, so that
 * moe_backward need not recompute them.  bf16 layers only (else
 * MOE_ERR_UNSUPPORTED).
 *   x_perm, perm_src, x, offsets as for moe_expert_up
 *   hidden [R, h] bf16 (out) as for moe_expert_up
 *   preact [R, N_up] bf16 (out): SwiGLU x W1^T (gate rows, columns 0..h-1)
 *          and x W3^T (up rows, columns h..2h-1); GELU x W1^T + b1 */
moe_status_t moe_expert_up_train(const moe_config_t *cfg, const moe_weights_t *w,
                                 const void *x_perm, const int32_t *perm_src,
                                 const void *x, const int32_t *offsets,
                                 void *hidden, void *preact, hipStream_t stream);

/* Down projection of every group: y_perm[r] = W2[e] hidden[r] (+ b2[e]).
 *   hidden [R, h] dtype (in), y_perm [R, d] dtype (out) */
moe_status_t moe_expert_down(const moe_config_t *cfg, const moe_weights_t *w,
                             const void *hidden, const int32_t *offsets,
                             void *y_perm, hipStream_t stream);

/* moe_expert_up then moe_expert_down, hidden rows in the workspace; the
 * token rows as for moe_expert_up (x_perm, or perm_src and x). */
moe_status_t moe_expert_ffn(const moe_config_t *cfg, const moe_weights_t *w,
                            const void *x_perm, const int32_t *perm_src,
                            const void *x, const int32_t *offsets, void *y_perm,
                            void *ws, size_t ws_bytes, hipStream_t stream);

/* Collect: y[t] = sum_{j<k} topk_w[t,j] * y_perm[pos[t*k+j]] (+ the shared
 * row y_perm[T*k + t] with weight 1), accumulated in fp32 in slot order and
 * rounded once to dtype (Go chapter section 2, Forward: out += w * y);
 * slots with pos = -1 (dropped by the capacity) are skipped.
 *   y_perm [R, d], pos [T*k], topk_w [T, k] (in); y [T, d] dtype (out) */
moe_status_t moe_combine(const moe_config_t *cfg, const void *y_perm,
                         const int32_t *pos, const float *topk_w, void *y,
                         hipStream_t stream);

/* The whole layer: route, permute, expert up/down, combine (the up
 * projection reads the token rows of x in place when T*d*bytes < 2^31).
 *   x [T, d] (in); y [T, d] (out); topk_idx, topk_w, counts, importance as
 *   above (out, required); stats [3] double or NULL (out). */
moe_status_t moe_forward(const moe_config_t *cfg, const moe_weights_t *w,
                         const void *x, void *y, int32_t *topk_idx,
                         float *topk_w, int32_t *counts, float *importance,
                         double *stats, void *ws, size_t ws_bytes,
                         hipStream_t stream);

/* Rewrites `count` row-major bf16 matrices [rows, cols] (src) into the
 * tiled order (dst, the same number of bytes) that moe_weights_t takes with
 * layout MOE_LAYOUT_TILED: the same expert matrices ("Weight Loading
 * Refactor" section of "Understanding MoE in Transformers"), stored so that
 * each 16-row x 32-column block is 1 KB of contiguous memory.  The stack of
 * count matrices is treated as one [count*rows, cols] matrix (rows is a
 * multiple of 16, so no block straddles two matrices).
 *   Block (rb, kb), rb < count*rows/16, kb < cols/32, is the 1 KB at byte
 *   offset (rb * cols/32 + kb) * 1024 of dst; its 16-byte piece p (0..63)
 *   holds row 16*rb + p/4, columns 32*kb + 8*c .. 32*kb + 8*c + 7, where
 *   c = (p % 4) XOR (p / 16).
 *   rows > 0, rows % 16 == 0, cols > 0, cols % 32 == 0, count >= 0 (0: no
 *   work), else MOE_ERR_INVALID_ARGUMENT; src and dst are device pointers,
 *   16-byte aligned, owned by the caller, and must not overlap
 *   (MOE_ERR_INVALID_ARGUMENT).  One kernel on `stream`; run it once when
 *   the weights are loaded, not per forward call. */
moe_status_t moe_tile_weights(const void *src, void *dst, int64_t count, int32_t rows,
                              int32_t cols, hipStream_t stream);

/* Backward pass: gradients of <dy, y> + importance_weight * CV^2(Importance)
 * with the top-k selection of the forward held fixed (the selection has no
 * derivative, so the router learns through the softmax weights only:
 * techfeed summary, "The hardest part: making the router trainable";
 * Importance and its CV^2: Qiita summary, "Load-balancing losses").  bf16 layers
 * in every gate mode: under MOE_GATE_BIAS_SELECTS the bias gets a zero
 * gradient; under MOE_GATE_SOFTMAX_ALL every score has a gradient (the gate
 * value of a kept expert is its share of the softmax over all E), so the
 * router gradients are dense and the backward reads the forward's scores.
 * An expert capacity is honoured through pos (a
 * dropped slot passes no gradient to its expert; its gate still counts in
 * Importance).  Every gradient has the dtype of its parameter: dx and the
 * expert weight and bias gradients bf16, the router's fp32 (accumulation is
 * fp32 throughout, one rounding at the end).
 *   x [T, d], dy [T, d]                  (device, in)
 *   saved from the forward (device, in): topk_idx, topk_w [T, k] (moe_route),
 *     offsets [E+1], pos [T*k], x_perm (moe_permute), y_perm [T*k + S*T, d]
 *     (the expert outputs, moe_expert_down / moe_expert_ffn)
 *   hidden [R, h], preact [R, N_up] bf16 or NULL (moe_expert_up_train's):
 *     when preact is NULL the pre-activations are recomputed (one more up
 *     projection); when hidden is NULL it is formed from the pre-activations
 *   logits [T, E] fp32 (moe_route's scores) under MOE_GATE_SOFTMAX_ALL,
 *     else ignored (may be NULL)
 *   noisy: NULL for the clean gate, else the noisy gate's values and the
 *     W_noise gradient (moe_noisy_grad_t, defined after moe_grads_t below;
 *     MOE_GATE_TOPK_SOFTMAX only)
 *   importance [E] fp32 or NULL (moe_permute's), importance_weight: the
 *     weight of the CV^2(Importance) term (ignored when importance is NULL)
 *   grads: every pointer device memory, written in full:
 *     dx [T, d] bf16; dw_gate [E, d] fp32; db_gate [E] fp32 or NULL; dw_up,
 *     dw_down bf16 with the shapes of w_up, w_down; db_up [E, h], db_down
 *     [E, d] bf16 or NULL (GELU); dw_up_shared [1, 2h, d], dw_down_shared
 *     [1, d, h] bf16 iff S = 1
 *   ws >= moe_backward_workspace_bytes(cfg) bytes (device, scratch)
 * Sums run in a fixed order: results are deterministic. */
typedef struct {
  void *dx;
  float *dw_gate;
  float *db_gate;
  void *dw_up;
  void *dw_down;
  void *db_up;
  void *db_down;
  void *dw_up_shared;
  void *dw_down_shared;
} moe_grads_t;

/* The noisy gate's share of the backward pass (the forward ran
 * moe_route_noisy): its gate values are the softmax of the kept noisy
 * scores H = s + n * Softplus(x W_noise^T), so the gradient reaches W_noise
 * too; with a load weight the loss also holds load_weight * CV^2(Load) of
 * the smooth Load (Qiita summary, "Load-balancing losses"), whose
 * thresholds are the forward's entries of H (the k-th, or for a kept
 * expert the (k+1)-th, of the stable descending order).
 *   w_noise [E, d] fp32, noise [T, E] fp32 (the draws), clean_logits and
 *   noise_scale [T, E] fp32, load [E] fp32 or NULL: moe_route_noisy's
 *   inputs and outputs (device, in)
 *   load_weight: the weight of CV^2(Load) (ignored when load is NULL)
 *   dw_noise [E, d] fp32 (device, out, written in full) */
typedef struct {
  const float *w_noise;
  const float *noise;
  const float *clean_logits;
  const float *noise_scale;
  const float *load;
  float load_weight;
  float *dw_noise;
} moe_noisy_grad_t;

/* Workspace bytes of moe_backward for cfg (bf16 layers), enough for every
 * gate mode and for the noisy gate (whose use the configuration does not
 * name).  Pure host; *bytes is 0 when T == 0. */
moe_status_t moe_backward_workspace_bytes(const moe_config_t *cfg, size_t *bytes);

moe_status_t moe_backward(const moe_config_t *cfg, const moe_weights_t *w,
                          const void *x, const void *dy, const int32_t *topk_idx,
                          const float *topk_w, const int32_t *offsets,
                          const int32_t *pos, const void *x_perm, const void *y_perm,
                          const void *hidden, const void *preact, const float *logits,
                          const moe_noisy_grad_t *noisy,
                          const float *importance, float importance_weight,
                          const moe_grads_t *grads, void *ws, size_t ws_bytes,
                          hipStream_t stream);

/* Host-only helpers. */

/* Parameter accounting of the Go chapter's section 1: Total = d*E + E*P_e,
 * Active = d*E + k*P_e, with P_e = 2*d*h (GELU) or 3*d*h (SwiGLU); a shared
 * expert adds P_e to both; biases are not counted. */
moe_status_t moe_param_counts(const moe_config_t *cfg, int64_t *total,
                              int64_t *active);

/* Expert capacity from a capacity factor: C = ceil(factor * T * k / E), at
 * least 1 (factor > 0; MOE_ERR_UNSUPPORTED if C would not fit int32). */
moe_status_t moe_expert_capacity(int64_t num_tokens, int32_t top_k, int32_t num_experts,
                                 double factor, int32_t *capacity);

/* Side statistics from host arrays: CV^2(importance), CV^2(counts) and the
 * load-balance loss E * sum_e (counts_e / sum counts)^2 (0 when the sum is
 * 0); population variance, CV^2 = 0 when the mean is 0.  importance may be
 * NULL (then *cv2_importance = 0). */
moe_status_t moe_load_stats(const int32_t *counts, const float *importance,
                            int32_t num_experts, double *cv2_importance,
                            double *cv2_load, double *load_balance);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */
