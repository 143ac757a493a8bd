// api.cpp - the C ABI (include/moe.h): argument checks, workspace carving and
// kernel launches.  Host code only; every kernel lives in the .hip files.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>

#include "moe.h"
#include "backward.h"
#include "permute.h"

namespace moe {
hipError_t launch_fill_i32(int32_t *p, int n, int32_t v, hipStream_t s);
hipError_t launch_route(bool bf16, int gate, const void *x, const float *wg, const float *bg,
                        int T, int d, int E, int k, int32_t *idx, float *w,
                        int32_t *counts, float *logits, hipStream_t s);
int64_t noisy_workspace_bytes(int64_t T, int E);
hipError_t launch_noisy_gate(const float *noise, int T, int E, int k, const float *clean,
                             float *scale, int32_t *idx, float *w, int32_t *counts,
                             float *importance, float *load, double *cv2, void *ws,
                             hipStream_t s);
hipError_t launch_expert_up_bf16(bool swiglu, const int32_t *offsets, int E, int S,
                                 int T, int k, int d, int h, const void *x_perm,
                                 const int32_t *perm_src, const void *x, const void *w_up,
                                 const void *w_up_shared, const void *b_up,
                                 void *hidden, bool w_tiled, hipStream_t s);
hipError_t launch_expert_up_train_bf16(bool swiglu, const int32_t *offsets, int E, int S,
                                       int T, int k, int d, int h, const void *x_perm,
                                       const int32_t *perm_src, const void *x,
                                       const void *w_up, const void *w_up_shared,
                                       const void *b_up, void *hidden, void *preact,
                                       bool w_tiled, hipStream_t s);
hipError_t launch_expert_down_bf16(const int32_t *offsets, int E, int S, int T, int k,
                                   int d, int h, const void *hidden,
                                   const void *w_down, const void *w_down_shared,
                                   const void *b_down, void *y_perm, bool w_tiled,
                                   hipStream_t s);
hipError_t launch_tile_weights(const void *src, void *dst, int64_t rows, int cols,
                               hipStream_t s);
hipError_t launch_expert_up_f32(bool swiglu, const int32_t *offsets, int E, int S,
                                int T, int k, int d, int h, const void *x_perm,
                                const int32_t *perm_src, const void *x, const void *w_up,
                                const void *w_up_shared, const void *b_up,
                                void *hidden, hipStream_t s);
hipError_t launch_expert_down_f32(const int32_t *offsets, int E, int S, int T, int k,
                                  int d, int h, const void *hidden,
                                  const void *w_down, const void *w_down_shared,
                                  const void *b_down, void *y_perm, hipStream_t s);
hipError_t launch_combine(bool bf16, const void *y_perm, const int32_t *pos,
                          const float *w, int T, int k, int d, int S, void *y,
                          hipStream_t s);
hipError_t launch_zero_stats(float *importance, int E, double *stats, hipStream_t s);
}  // namespace moe

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool dev_ok(const void *p) { return p != nullptr && aligned16(p); }
bool opt_ok(const void *p) { return p == nullptr || aligned16(p); }

moe_status_t check_cfg(const moe_config_t *c) {
  if (!c) return MOE_ERR_INVALID_ARGUMENT;
  if (c->num_tokens < 0 || c->d_model <= 0 || c->d_hidden <= 0 ||
      c->num_experts < 1 || c->top_k < 1 || c->top_k > c->num_experts ||
      c->num_shared < 0 || c->capacity < 0 || c->gate < MOE_GATE_TOPK_SOFTMAX ||
      c->gate > MOE_GATE_SOFTMAX_ALL || c->overflow < MOE_OVERFLOW_DROP ||
      c->overflow > MOE_OVERFLOW_NEXT_CHOICE)
    return MOE_ERR_INVALID_ARGUMENT;
  if ((c->act != MOE_ACT_GELU && c->act != MOE_ACT_SWIGLU) ||
      (c->dtype != MOE_DTYPE_F32 && c->dtype != MOE_DTYPE_BF16))
    return MOE_ERR_INVALID_ARGUMENT;
  if (c->num_experts > 256 || c->num_shared > 1) return MOE_ERR_UNSUPPORTED;
  if (c->num_shared == 1 && c->act != MOE_ACT_SWIGLU) return MOE_ERR_UNSUPPORTED;
  if (c->d_model % 64 != 0 || c->d_hidden % 64 != 0) return MOE_ERR_UNSUPPORTED;
  const int64_t rows = c->num_tokens * (c->top_k + c->num_shared);
  if (rows >= (int64_t(1) << 31)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

moe_status_t check_weights(const moe_config_t *c, const moe_weights_t *w, bool up,
                           bool down, bool router) {
  if (!w) return MOE_ERR_INVALID_ARGUMENT;
  if (w->layout != MOE_LAYOUT_ROW_MAJOR && w->layout != MOE_LAYOUT_TILED)
    return MOE_ERR_INVALID_ARGUMENT;
  if (w->layout == MOE_LAYOUT_TILED && c->dtype != MOE_DTYPE_BF16) return MOE_ERR_UNSUPPORTED;
  if (router && !dev_ok(w->w_gate)) return MOE_ERR_INVALID_ARGUMENT;
  if (router && !opt_ok(w->b_gate)) return MOE_ERR_INVALID_ARGUMENT;
  const bool swi = c->act == MOE_ACT_SWIGLU;
  if (up) {
    if (!dev_ok(w->w_up) || !opt_ok(w->b_up)) return MOE_ERR_INVALID_ARGUMENT;
    if (swi && w->b_up) return MOE_ERR_INVALID_ARGUMENT;
    if (c->num_shared ? !dev_ok(w->w_up_shared) : w->w_up_shared != nullptr)
      return MOE_ERR_INVALID_ARGUMENT;
  }
  if (down) {
    if (!dev_ok(w->w_down) || !opt_ok(w->b_down)) return MOE_ERR_INVALID_ARGUMENT;
    if (swi && w->b_down) return MOE_ERR_INVALID_ARGUMENT;
    if (c->num_shared ? !dev_ok(w->w_down_shared) : w->w_down_shared != nullptr)
      return MOE_ERR_INVALID_ARGUMENT;
  }
  return MOE_OK;
}

size_t elem_bytes(const moe_config_t *c) { return c->dtype == MOE_DTYPE_BF16 ? 2 : 4; }

// Workspace regions, each 256-byte aligned, in this order.
struct Layout {
  size_t hist, full_off, perm_w;                        // moe_permute scratch
  size_t pos_a, cand, pos_b, fin, off_b, full_off_b, permute_end;  // re-routing
  size_t offsets, perm_src, pos, logits, x_perm, hidden, y_perm, total;  // moe_forward
};

bool reroutes(const moe_config_t *c) {
  return c->capacity > 0 && c->overflow == MOE_OVERFLOW_NEXT_CHOICE;
}

// moe_forward reads the token rows of the up projection from x in place
// (no grouped copy) whenever 32-bit byte offsets reach every row of x.
bool gathers(const moe_config_t *c) {
  return (uint64_t)c->num_tokens * c->d_model * (c->dtype == MOE_DTYPE_BF16 ? 2 : 4) <
         (1ull << 31);
}

Layout layout(const moe_config_t *c) {
  const int64_t T = c->num_tokens, n = T * c->top_k;
  const int64_t R = n + (int64_t)c->num_shared * T;
  const size_t es = elem_bytes(c);
  const int E = c->num_experts;
  Layout L{};
  size_t o = 0;
  L.hist = o;      o += align_up(sizeof(int32_t) * (size_t)moe::perm_num_segments(n) * E);
  L.full_off = o;  o += align_up(sizeof(int32_t) * (size_t)(E + 1));
  L.perm_w = o;    o += align_up(sizeof(float) * (size_t)n);
  const size_t rn = reroutes(c) ? (size_t)n : 0, re = reroutes(c) ? (size_t)E : 0;
  L.pos_a = o;       o += align_up(sizeof(int32_t) * rn);
  L.cand = o;        o += align_up(sizeof(int32_t) * rn);
  L.pos_b = o;       o += align_up(sizeof(int32_t) * rn);
  L.fin = o;         o += align_up(sizeof(int32_t) * rn);
  L.off_b = o;       o += align_up(sizeof(int32_t) * (re ? re + 1 : 0));
  L.full_off_b = o;  o += align_up(sizeof(int32_t) * (re ? re + 1 : 0));
  L.permute_end = o;
  L.offsets = o;   o += align_up(sizeof(int32_t) * (size_t)(E + 1));
  L.perm_src = o;  o += align_up(sizeof(int32_t) * (size_t)n);
  L.pos = o;       o += align_up(sizeof(int32_t) * (size_t)n);
  L.logits = o;    o += align_up(sizeof(float) * (reroutes(c) ? (size_t)T * E : 0));
  L.x_perm = o;    o += align_up(gathers(c) ? 0 : es * (size_t)n * c->d_model);
  L.hidden = o;    o += align_up(es * (size_t)R * c->d_hidden);
  L.y_perm = o;    o += align_up(es * (size_t)R * c->d_model);
  L.total = o;
  // moe_route_noisy uses the front of the workspace for its partial sums
  const size_t noisy = align_up((size_t)moe::noisy_workspace_bytes(T, E));
  if (L.total < noisy) L.total = noisy;
  return L;
}

size_t hidden_bytes(const moe_config_t *c) {
  const int64_t R = c->num_tokens * (c->top_k + c->num_shared);
  return align_up(elem_bytes(c) * (size_t)R * c->d_hidden);
}

template <typename T>
T *at(void *ws, size_t off) {
  return reinterpret_cast<T *>(static_cast<char *>(ws) + off);
}

moe_status_t hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// Pending errors of earlier, unrelated HIP calls are cleared so that a
// launch status reflects this call only.
void clear_pending_error() { (void)hipGetLastError(); }

// Backward workspace regions, each 256-byte aligned, in this order.
struct BwdLayout {
  size_t gimp, ds, poff, colsrc;
  size_t A, H, dyp, dH, dA, dxp, dypT, HT, dAT, xpT;
  size_t tm, dS, dU, gload, dxr, dpart, total;
};

BwdLayout bwd_layout(const moe_config_t *c) {
  const int64_t T = c->num_tokens, k = c->top_k, E = c->num_experts, S = c->num_shared;
  const int64_t d = c->d_model, h = c->d_hidden;
  const int64_t nup = c->act == MOE_ACT_SWIGLU ? 2 * h : h;
  const int64_t R = T * k + S * T;
  const int64_t Rp = moe::bwd_padded_cols(T, (int)k, (int)E, (int)S);
  BwdLayout L{};
  size_t o = 0;
  auto take = [&](size_t &f, int64_t bytes) {
    f = o;
    o += align_up((size_t)bytes);
  };
  take(L.gimp, 4 * E);
  take(L.ds, 4 * T * k);
  take(L.poff, 4 * (E + S + 1));
  take(L.colsrc, 4 * Rp);
  take(L.A, 2 * R * nup);
  take(L.H, 2 * R * h);
  take(L.dyp, 2 * R * d);
  take(L.dH, 2 * R * h);
  take(L.dA, 2 * R * nup);
  take(L.dxp, 2 * R * d);
  take(L.dypT, 2 * d * Rp);
  take(L.HT, 2 * h * Rp);
  take(L.dAT, 2 * nup * Rp);
  take(L.xpT, 2 * d * Rp);
  // router gradients: the dense score gradients of every gate; the dense
  // share of dx and the noise-score gradients of the softmax-all and noisy
  // gates (the configuration does not name the noisy gate, so the space is
  // always there)
  take(L.tm, 4 * T);
  take(L.dS, 4 * T * E);
  take(L.dU, 4 * T * E);
  take(L.gload, 4 * E);
  take(L.dxr, 4 * T * d);
  int splits = 1, kchunk = 0;
  if (T > 0) moe::bwd_dense_plan(T, (int)E, (int)d, &splits, &kchunk);
  take(L.dpart, splits > 1 ? 4 * (int64_t)splits * E * d : 0);
  L.total = o;
  return L;
}

moe_status_t check_bwd_cfg(const moe_config_t *cfg) {
  moe_status_t st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  if (cfg->dtype != MOE_DTYPE_BF16) return MOE_ERR_UNSUPPORTED;
  const int64_t Rp = moe::bwd_padded_cols(cfg->num_tokens, cfg->top_k, cfg->num_experts,
                                          cfg->num_shared);
  if (Rp >= (int64_t(1) << 31) / 512) return MOE_ERR_UNSUPPORTED;   // 32-bit tile offsets
  return MOE_OK;
}


}  // namespace

extern "C" {

int moe_abi_version(void) { return MOE_ABI_VERSION; }

const char *moe_status_string(moe_status_t s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARGUMENT: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported configuration";
    case MOE_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case MOE_ERR_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

moe_status_t moe_workspace_bytes(const moe_config_t *cfg, size_t *bytes) {
  moe_status_t st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  if (!bytes) return MOE_ERR_INVALID_ARGUMENT;
  *bytes = cfg->num_tokens == 0 ? 0 : layout(cfg).total;
  return MOE_OK;
}

moe_status_t moe_grouped_rows(const moe_config_t *cfg, int64_t *rows) {
  moe_status_t st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  if (!rows) return MOE_ERR_INVALID_ARGUMENT;
  *rows = cfg->num_tokens * (cfg->top_k + cfg->num_shared);
  return MOE_OK;
}

moe_status_t moe_route(const moe_config_t *cfg, const void *x, const float *w_gate,
                       const float *b_gate, int32_t *topk_idx, float *topk_w,
                       int32_t *counts, float *logits, hipStream_t stream) {
  moe_status_t st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  if (!opt_ok(counts)) return MOE_ERR_INVALID_ARGUMENT;
  const int T = (int)cfg->num_tokens;
  if (T > 0 && (!dev_ok(x) || !dev_ok(w_gate) || !opt_ok(b_gate) ||
                !dev_ok(topk_idx) || !dev_ok(topk_w) || !opt_ok(logits)))
    return MOE_ERR_INVALID_ARGUMENT;
  clear_pending_error();
  return hip_status(moe::launch_route(cfg->dtype == MOE_DTYPE_BF16, cfg->gate, x, w_gate,
                                      b_gate, T,
                                      cfg->d_model, cfg->num_experts, cfg->top_k,
                                      topk_idx, topk_w, counts, logits, stream));
}

moe_status_t moe_route_noisy(const moe_config_t *cfg, const void *x, const float *w_gate,
                             const float *b_gate, const float *w_noise, const float *noise,
                             float *clean_logits, float *noise_scale, int32_t *topk_idx,
                             float *topk_w, int32_t *counts, float *importance, float *load,
                             double *cv2, void *workspace, size_t workspace_bytes,
                             hipStream_t stream) {
  moe_status_t st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  if (cfg->gate != MOE_GATE_TOPK_SOFTMAX) return MOE_ERR_UNSUPPORTED;
  if (!dev_ok(counts) || !dev_ok(importance) || !dev_ok(load) || !opt_ok(cv2))
    return MOE_ERR_INVALID_ARGUMENT;
  const int T = (int)cfg->num_tokens, E = cfg->num_experts;
  if (T > 0 && (!dev_ok(x) || !dev_ok(w_gate) || !opt_ok(b_gate) || !dev_ok(w_noise) ||
                !dev_ok(noise) || !dev_ok(clean_logits) || !dev_ok(noise_scale) ||
                !dev_ok(topk_idx) || !dev_ok(topk_w)))
    return MOE_ERR_INVALID_ARGUMENT;
  const size_t need = (size_t)moe::noisy_workspace_bytes(T, E);
  if (T > 0 && !dev_ok(workspace)) return MOE_ERR_INVALID_ARGUMENT;
  if (T > 0 && workspace_bytes < need) return MOE_ERR_WORKSPACE_TOO_SMALL;
  clear_pending_error();
  const bool bf16 = cfg->dtype == MOE_DTYPE_BF16;
  hipError_t e = hipSuccess;
  if (T > 0) {
    // the router chains: raw noise scores into noise_scale, clean scores
    // (with the bias) into clean_logits; the indices, weights and counts
    // they also write are replaced by the noisy gate below
    e = moe::launch_route(bf16, MOE_GATE_TOPK_SOFTMAX, x, w_noise, nullptr, T, cfg->d_model,
                          E, cfg->top_k, topk_idx, topk_w, counts, noise_scale, stream);
    if (e == hipSuccess)
      e = moe::launch_route(bf16, MOE_GATE_TOPK_SOFTMAX, x, w_gate, b_gate, T, cfg->d_model,
                            E, cfg->top_k, topk_idx, topk_w, counts, clean_logits, stream);
  }
  if (e == hipSuccess)
    e = moe::launch_noisy_gate(noise, T, E, cfg->top_k, clean_logits, noise_scale, topk_idx,
                               topk_w, counts, importance, load, cv2,
                               T > 0 ? workspace : nullptr, stream);
  return hip_status(e);
}

}  // extern "C"

namespace {

// moe_permute; counts_out (or NULL): the assignments per expert from the
// grouping's histogram (moe_forward takes the counts from here instead of
// zeroing and accumulating them in the router)
moe_status_t permute_impl(const moe_config_t *cfg, const int32_t *topk_idx,
                          const float *topk_w, const float *logits, const void *x,
                          int32_t *offsets, int32_t *perm_src, int32_t *pos, float *importance,
                          double *stats, void *x_perm, void *ws, size_t ws_bytes,
                          hipStream_t stream, int32_t *counts_out) {
  moe_status_t st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  const int T = (int)cfg->num_tokens;
  if (!dev_ok(offsets) || !dev_ok(importance) || !opt_ok(stats) || !opt_ok(counts_out))
    return MOE_ERR_INVALID_ARGUMENT;
  if (T > 0 && (!dev_ok(topk_idx) || !dev_ok(topk_w) || !dev_ok(x) ||
                !dev_ok(perm_src) || !dev_ok(pos) || !opt_ok(x_perm) || !dev_ok(ws) ||
                (reroutes(cfg) && !dev_ok(logits))))
    return MOE_ERR_INVALID_ARGUMENT;
  const Layout L = layout(cfg);
  if (T > 0 && ws_bytes < L.permute_end) return MOE_ERR_WORKSPACE_TOO_SMALL;
  clear_pending_error();
  if (T == 0) {
    hipError_t e = moe::launch_fill_i32(offsets, cfg->num_experts + 1, 0, stream);
    if (e == hipSuccess && counts_out)
      e = moe::launch_fill_i32(counts_out, cfg->num_experts, 0, stream);
    if (e != hipSuccess) return MOE_ERR_HIP;
  }
  if (T > 0 && reroutes(cfg)) {
    moe::RerouteScratch r{at<int32_t>(ws, L.pos_a),  at<int32_t>(ws, L.cand),
                          at<int32_t>(ws, L.pos_b),  at<int32_t>(ws, L.fin),
                          at<int32_t>(ws, L.off_b),  at<int32_t>(ws, L.full_off_b)};
    return hip_status(moe::launch_permute_reroute(
        topk_idx, topk_w, logits, x, T, cfg->top_k, cfg->num_experts, cfg->capacity,
        (int)(cfg->d_model * elem_bytes(cfg)), offsets, perm_src, pos, importance, stats,
        x_perm, at<int32_t>(ws, L.hist), at<int32_t>(ws, L.full_off), at<float>(ws, L.perm_w),
        r, stream, counts_out));
  }
  return hip_status(moe::launch_permute(
      topk_idx, topk_w, x, T, cfg->top_k, cfg->num_experts, cfg->capacity,
      (int)(cfg->d_model * elem_bytes(cfg)), offsets, perm_src, pos, importance, stats,
      x_perm, T ? at<int32_t>(ws, L.hist) : nullptr, T ? at<int32_t>(ws, L.full_off) : nullptr,
      T ? at<float>(ws, L.perm_w) : nullptr, stream, counts_out));
}

}  // namespace

extern "C" {

moe_status_t moe_permute(const moe_config_t *cfg, const int32_t *topk_idx,
                         const float *topk_w, const float *logits, const void *x,
                         int32_t *offsets,
                         int32_t *perm_src, int32_t *pos, float *importance,
                         double *stats, int32_t *counts, void *x_perm, void *ws,
                         size_t ws_bytes, hipStream_t stream) {
  return permute_impl(cfg, topk_idx, topk_w, logits, x, offsets, perm_src, pos, importance,
                      stats, x_perm, ws, ws_bytes, stream, counts);
}

// The token rows of the up projection: x_perm (the grouped copy), or, when
// x_perm is NULL, rows perm_src[p] of x read in place.  The gathered rows are
// addressed with 32-bit byte offsets into x.
moe_status_t check_up_rows(const moe_config_t *cfg, const void *x_perm,
                           const int32_t *perm_src, const void *x) {
  if (x_perm) return dev_ok(x_perm) && (!cfg->num_shared || dev_ok(x)) ? MOE_OK
                                                                     : MOE_ERR_INVALID_ARGUMENT;
  if (!dev_ok(perm_src) || !dev_ok(x)) return MOE_ERR_INVALID_ARGUMENT;
  if ((uint64_t)cfg->num_tokens * cfg->d_model * elem_bytes(cfg) >= (1ull << 31))
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

static_assert(MOE_NOALLOC_SCRATCH_BYTES == moe::kNoallocScratchBytes,
              "the header states the static scratch size");

moe_status_t moe_permute_noalloc(const moe_config_t *cfg, const int32_t *topk_idx,
                                 const float *topk_w, const float *logits, const void *x,
                                 int32_t *offsets, int32_t *perm_src, int32_t *pos,
                                 float *importance, double *stats, int32_t *counts,
                                 void *x_perm, hipStream_t stream) {
  moe_status_t st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  // the scratch this configuration needs must fit the static array (checked
  // on the host, before any device call)
  if (cfg->num_tokens > 0 && layout(cfg).permute_end > moe::kNoallocScratchBytes)
    return MOE_ERR_WORKSPACE_TOO_SMALL;
  void *ws = nullptr;
  if (cfg->num_tokens > 0) {
    clear_pending_error();
    if (moe::noalloc_scratch(&ws) != hipSuccess) return MOE_ERR_HIP;
  }
  return permute_impl(cfg, topk_idx, topk_w, logits, x, offsets, perm_src, pos, importance,
                      stats, x_perm, ws, ws ? moe::kNoallocScratchBytes : 0, stream, counts);
}

moe_status_t moe_expert_up(const moe_config_t *cfg, const moe_weights_t *w,
                           const void *x_perm, const int32_t *perm_src, const void *x,
                           const int32_t *offsets, void *hidden, hipStream_t stream) {
  moe_status_t st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  if ((st = check_weights(cfg, w, true, false, false)) != MOE_OK) return st;
  const int T = (int)cfg->num_tokens;
  if (T == 0) return MOE_OK;
  if (!dev_ok(offsets) || !dev_ok(hidden)) return MOE_ERR_INVALID_ARGUMENT;
  if ((st = check_up_rows(cfg, x_perm, perm_src, x)) != MOE_OK) return st;
  clear_pending_error();
  const bool swi = cfg->act == MOE_ACT_SWIGLU;
  if (cfg->dtype == MOE_DTYPE_BF16)
    return hip_status(moe::launch_expert_up_bf16(
        swi, offsets, cfg->num_experts, cfg->num_shared, T, cfg->top_k, cfg->d_model,
        cfg->d_hidden, x_perm, perm_src, x, w->w_up, w->w_up_shared, w->b_up, hidden,
        w->layout == MOE_LAYOUT_TILED, stream));
  return hip_status(moe::launch_expert_up_f32(
      swi, offsets, cfg->num_experts, cfg->num_shared, T, cfg->top_k, cfg->d_model,
      cfg->d_hidden, x_perm, perm_src, x, w->w_up, w->w_up_shared, w->b_up, hidden, stream));
}

moe_status_t moe_expert_up_train(const moe_config_t *cfg, const moe_weights_t *w,
                                 const void *x_perm, const int32_t *perm_src, const void *x,
                                 const int32_t *offsets, void *hidden, void *preact,
                                 hipStream_t stream) {
  moe_status_t st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  if (cfg->dtype != MOE_DTYPE_BF16) return MOE_ERR_UNSUPPORTED;
  if ((st = check_weights(cfg, w, true, false, false)) != MOE_OK) return st;
  const int T = (int)cfg->num_tokens;
  if (T == 0) return MOE_OK;
  if (!dev_ok(offsets) || !dev_ok(hidden) || !dev_ok(preact)) return MOE_ERR_INVALID_ARGUMENT;
  if ((st = check_up_rows(cfg, x_perm, perm_src, x)) != MOE_OK) return st;
  clear_pending_error();
  return hip_status(moe::launch_expert_up_train_bf16(
      cfg->act == MOE_ACT_SWIGLU, offsets, cfg->num_experts, cfg->num_shared, T, cfg->top_k,
      cfg->d_model, cfg->d_hidden, x_perm, perm_src, x, w->w_up, w->w_up_shared, w->b_up,
      hidden, preact, w->layout == MOE_LAYOUT_TILED, stream));
}

moe_status_t moe_expert_down(const moe_config_t *cfg, const moe_weights_t *w,
                             const void *hidden, const int32_t *offsets, void *y_perm,
                             hipStream_t stream) {
  moe_status_t st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  if ((st = check_weights(cfg, w, false, true, false)) != MOE_OK) return st;
  const int T = (int)cfg->num_tokens;
  if (T == 0) return MOE_OK;
  if (!dev_ok(hidden) || !dev_ok(offsets) || !dev_ok(y_perm))
    return MOE_ERR_INVALID_ARGUMENT;
  clear_pending_error();
  if (cfg->dtype == MOE_DTYPE_BF16)
    return hip_status(moe::launch_expert_down_bf16(
        offsets, cfg->num_experts, cfg->num_shared, T, cfg->top_k, cfg->d_model,
        cfg->d_hidden, hidden, w->w_down, w->w_down_shared, w->b_down, y_perm,
        w->layout == MOE_LAYOUT_TILED, stream));
  return hip_status(moe::launch_expert_down_f32(
      offsets, cfg->num_experts, cfg->num_shared, T, cfg->top_k, cfg->d_model,
      cfg->d_hidden, hidden, w->w_down, w->w_down_shared, w->b_down, y_perm, stream));
}

moe_status_t moe_expert_ffn(const moe_config_t *cfg, const moe_weights_t *w,
                            const void *x_perm, const int32_t *perm_src, const void *x,
                            const int32_t *offsets, void *y_perm, void *ws, size_t ws_bytes,
                            hipStream_t stream) {
  moe_status_t st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  if ((st = check_weights(cfg, w, true, true, false)) != MOE_OK) return st;
  if (cfg->num_tokens == 0) return MOE_OK;
  if (!dev_ok(ws)) return MOE_ERR_INVALID_ARGUMENT;
  if (ws_bytes < hidden_bytes(cfg)) return MOE_ERR_WORKSPACE_TOO_SMALL;
  if (!dev_ok(offsets) || !dev_ok(y_perm)) return MOE_ERR_INVALID_ARGUMENT;
  if ((st = check_up_rows(cfg, x_perm, perm_src, x)) != MOE_OK) return st;
  if ((st = moe_expert_up(cfg, w, x_perm, perm_src, x, offsets, ws, stream)) != MOE_OK)
    return st;
  return moe_expert_down(cfg, w, ws, offsets, y_perm, stream);
}

moe_status_t moe_combine(const moe_config_t *cfg, const void *y_perm, const int32_t *pos,
                         const float *topk_w, void *y, hipStream_t stream) {
  moe_status_t st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  const int T = (int)cfg->num_tokens;
  if (T == 0) return MOE_OK;
  if (!dev_ok(y_perm) || !dev_ok(pos) || !dev_ok(topk_w) || !dev_ok(y))
    return MOE_ERR_INVALID_ARGUMENT;
  clear_pending_error();
  return hip_status(moe::launch_combine(cfg->dtype == MOE_DTYPE_BF16, y_perm, pos,
                                            topk_w, T, cfg->top_k, cfg->d_model,
                                            cfg->num_shared, y, stream));
}

moe_status_t moe_forward(const moe_config_t *cfg, const moe_weights_t *w, const void *x,
                         void *y, int32_t *topk_idx, float *topk_w, int32_t *counts,
                         float *importance, double *stats, void *ws, size_t ws_bytes,
                         hipStream_t stream) {
  moe_status_t st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  if ((st = check_weights(cfg, w, true, true, true)) != MOE_OK) return st;
  const int T = (int)cfg->num_tokens;
  if (!dev_ok(counts) || !dev_ok(importance) || !opt_ok(stats))
    return MOE_ERR_INVALID_ARGUMENT;
  if (T > 0 && (!dev_ok(x) || !dev_ok(y) || !dev_ok(topk_idx) || !dev_ok(topk_w) ||
                !dev_ok(ws)))
    return MOE_ERR_INVALID_ARGUMENT;
  const Layout L = layout(cfg);
  if (T > 0 && ws_bytes < L.total) return MOE_ERR_WORKSPACE_TOO_SMALL;
  if (T == 0) {
    if ((st = moe_route(cfg, x, w->w_gate, w->b_gate, topk_idx, topk_w, counts, nullptr,
                        stream)) != MOE_OK)
      return st;
    clear_pending_error();
    return hip_status(moe::launch_zero_stats(importance, cfg->num_experts, stats, stream));
  }
  int32_t *offsets = at<int32_t>(ws, L.offsets);
  int32_t *perm_src = at<int32_t>(ws, L.perm_src);
  int32_t *pos = at<int32_t>(ws, L.pos);
  void *x_perm = gathers(cfg) ? nullptr : at<char>(ws, L.x_perm);
  void *hidden = at<char>(ws, L.hidden);
  void *y_perm = at<char>(ws, L.y_perm);
  float *logits = reroutes(cfg) ? at<float>(ws, L.logits) : nullptr;   // next choices
  // the router without counts: the grouping's histogram gives them
  if ((st = moe_route(cfg, x, w->w_gate, w->b_gate, topk_idx, topk_w, nullptr, logits,
                      stream)) != MOE_OK)
    return st;
  if ((st = permute_impl(cfg, topk_idx, topk_w, logits, x, offsets, perm_src, pos, importance,
                         stats, x_perm, ws, L.permute_end, stream, counts)) != MOE_OK)
    return st;
  if ((st = moe_expert_up(cfg, w, x_perm, perm_src, x, offsets, hidden, stream)) != MOE_OK)
    return st;
  if ((st = moe_expert_down(cfg, w, hidden, offsets, y_perm, stream)) != MOE_OK) return st;
  return moe_combine(cfg, y_perm, pos, topk_w, y, stream);
}

moe_status_t moe_tile_weights(const void *src, void *dst, int64_t count, int32_t rows,
                              int32_t cols, hipStream_t stream) {
  if (count < 0 || rows <= 0 || rows % 16 != 0 || cols <= 0 || cols % 32 != 0)
    return MOE_ERR_INVALID_ARGUMENT;
  if (count == 0) return MOE_OK;
  if (!dev_ok(src) || !dev_ok(dst)) return MOE_ERR_INVALID_ARGUMENT;
  if (count > INT64_MAX / rows / cols / 2) return MOE_ERR_INVALID_ARGUMENT;
  const uint64_t bytes = (uint64_t)count * rows * cols * 2;
  const uintptr_t s0 = reinterpret_cast<uintptr_t>(src), d0 = reinterpret_cast<uintptr_t>(dst);
  if (s0 < d0 + bytes && d0 < s0 + bytes) return MOE_ERR_INVALID_ARGUMENT;   // overlap
  clear_pending_error();
  return hip_status(moe::launch_tile_weights(src, dst, count * rows, cols, stream));
}

moe_status_t moe_backward_workspace_bytes(const moe_config_t *cfg, size_t *bytes) {
  moe_status_t st = check_bwd_cfg(cfg);
  if (st != MOE_OK) return st;
  if (!bytes) return MOE_ERR_INVALID_ARGUMENT;
  *bytes = cfg->num_tokens == 0 ? 0 : bwd_layout(cfg).total;
  return MOE_OK;
}

moe_status_t moe_backward(const moe_config_t *cfg, const moe_weights_t *w, const void *x,
                          const void *dy, const int32_t *topk_idx, const float *topk_w,
                          const int32_t *offsets, const int32_t *pos, const void *x_perm,
                          const void *y_perm, const void *hidden, const void *preact,
                          const float *logits, const moe_noisy_grad_t *noisy,
                          const float *importance,
                          float importance_weight, const moe_grads_t *g, void *ws,
                          size_t ws_bytes, hipStream_t stream) {
  moe_status_t st = check_bwd_cfg(cfg);
  if (st != MOE_OK) return st;
  if ((st = check_weights(cfg, w, true, true, true)) != MOE_OK) return st;
  // the backward's GEMMs read the expert matrices row-major only
  if (w->layout != MOE_LAYOUT_ROW_MAJOR) return MOE_ERR_UNSUPPORTED;
  if (!g || !dev_ok(g->dw_gate) || !dev_ok(g->dw_up) || !dev_ok(g->dw_down) ||
      !opt_ok(g->db_gate) || !opt_ok(g->db_up) || !opt_ok(g->db_down) ||
      !opt_ok(importance) || !opt_ok(hidden) || !opt_ok(preact) || !opt_ok(logits) ||
      !std::isfinite(importance_weight))
    return MOE_ERR_INVALID_ARGUMENT;
  const bool softmax_all = cfg->gate == MOE_GATE_SOFTMAX_ALL;
  if (noisy && (cfg->gate != MOE_GATE_TOPK_SOFTMAX || !dev_ok(noisy->w_noise) ||
                !dev_ok(noisy->dw_noise) || !opt_ok(noisy->load) ||
                !std::isfinite(noisy->load_weight)))
    return MOE_ERR_INVALID_ARGUMENT;
  const bool swi = cfg->act == MOE_ACT_SWIGLU;
  if (swi && (g->db_up || g->db_down)) return MOE_ERR_INVALID_ARGUMENT;
  if (cfg->num_shared ? (!dev_ok(g->dw_up_shared) || !dev_ok(g->dw_down_shared))
                      : (g->dw_up_shared || g->dw_down_shared))
    return MOE_ERR_INVALID_ARGUMENT;
  const int64_t T = cfg->num_tokens;
  const int E = cfg->num_experts, S = cfg->num_shared;
  const int64_t d = cfg->d_model, h = cfg->d_hidden, nup = swi ? 2 * h : h;
  clear_pending_error();
  if (T == 0) {
    hipError_t e = moe::launch_fill_f32(g->dw_gate, E * d, stream);
    if (e == hipSuccess && noisy) e = moe::launch_fill_f32(noisy->dw_noise, E * d, stream);
    if (e == hipSuccess) e = moe::launch_fill_f32(g->db_gate, E, stream);
    // bf16 gradients: a zero bf16 is two zero bytes; every count is even
    auto zero16 = [&](void *p, int64_t n) {
      return moe::launch_fill_f32(static_cast<float *>(p), n / 2, stream);
    };
    if (e == hipSuccess) e = zero16(g->dw_up, E * nup * d);
    if (e == hipSuccess) e = zero16(g->dw_down, E * d * h);
    if (e == hipSuccess) e = zero16(g->db_up, E * h);
    if (e == hipSuccess) e = zero16(g->db_down, E * d);
    if (e == hipSuccess) e = zero16(g->dw_up_shared, S * nup * d);
    if (e == hipSuccess) e = zero16(g->dw_down_shared, S * d * h);
    return hip_status(e);
  }
  if (!dev_ok(x) || !dev_ok(dy) || !dev_ok(topk_idx) || !dev_ok(topk_w) || !dev_ok(offsets) ||
      !dev_ok(pos) || !dev_ok(x_perm) || !dev_ok(y_perm) || !dev_ok(g->dx) ||
      (softmax_all && !dev_ok(logits)) ||
      (noisy && (!dev_ok(noisy->noise) || !dev_ok(noisy->clean_logits) ||
                 !dev_ok(noisy->noise_scale))))
    return MOE_ERR_INVALID_ARGUMENT;
  const BwdLayout L = bwd_layout(cfg);
  if (!dev_ok(ws)) return MOE_ERR_INVALID_ARGUMENT;
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE_TOO_SMALL;
  moe::BwdArgs a{};
  a.T = (int)T;
  a.k = cfg->top_k;
  a.E = E;
  a.S = S;
  a.d = (int)d;
  a.h = (int)h;
  a.swiglu = swi;
  a.capacity = cfg->capacity;
  a.bias_selects = cfg->gate == MOE_GATE_BIAS_SELECTS;
  a.x = static_cast<const uint16_t *>(x);
  a.dy = static_cast<const uint16_t *>(dy);
  a.w_up = static_cast<const uint16_t *>(w->w_up);
  a.w_down = static_cast<const uint16_t *>(w->w_down);
  a.b_up = static_cast<const uint16_t *>(w->b_up);
  a.w_up_s = static_cast<const uint16_t *>(w->w_up_shared);
  a.w_down_s = static_cast<const uint16_t *>(w->w_down_shared);
  a.w_gate = w->w_gate;
  a.idx = topk_idx;
  a.offsets = offsets;
  a.pos = pos;
  a.topk_w = topk_w;
  a.importance = importance;
  a.w_imp = importance_weight;
  a.x_perm = static_cast<const uint16_t *>(x_perm);
  a.y_perm = static_cast<const uint16_t *>(y_perm);
  a.hidden = static_cast<const uint16_t *>(hidden);
  a.preact = static_cast<const uint16_t *>(preact);
  a.logits = softmax_all ? logits : nullptr;
  if (noisy) {
    a.clean = noisy->clean_logits;
    a.scale = noisy->noise_scale;
    a.noise = noisy->noise;
    a.load = noisy->load;
    a.w_load = noisy->load_weight;
    a.w_noise = noisy->w_noise;
    a.dw_noise = noisy->dw_noise;
  }
  a.dx = static_cast<uint16_t *>(g->dx);
  a.dw_gate = g->dw_gate;
  a.db_gate = g->db_gate;
  a.dw_up = static_cast<uint16_t *>(g->dw_up);
  a.dw_down = static_cast<uint16_t *>(g->dw_down);
  a.db_up = static_cast<uint16_t *>(g->db_up);
  a.db_down = static_cast<uint16_t *>(g->db_down);
  a.dw_up_s = static_cast<uint16_t *>(g->dw_up_shared);
  a.dw_down_s = static_cast<uint16_t *>(g->dw_down_shared);
  moe::BwdBuffers b{};
  b.gimp = at<float>(ws, L.gimp);
  b.ds = at<float>(ws, L.ds);
  b.poff = at<int32_t>(ws, L.poff);
  b.colsrc = at<int32_t>(ws, L.colsrc);
  b.A = at<uint16_t>(ws, L.A);
  b.H = at<uint16_t>(ws, L.H);
  b.dyp = at<uint16_t>(ws, L.dyp);
  b.dH = at<uint16_t>(ws, L.dH);
  b.dA = at<uint16_t>(ws, L.dA);
  b.dxp = at<uint16_t>(ws, L.dxp);
  b.dypT = at<uint16_t>(ws, L.dypT);
  b.HT = at<uint16_t>(ws, L.HT);
  b.dAT = at<uint16_t>(ws, L.dAT);
  b.xpT = at<uint16_t>(ws, L.xpT);
  b.tm = at<float>(ws, L.tm);
  b.dS = at<float>(ws, L.dS);
  b.dU = at<float>(ws, L.dU);
  b.gload = at<float>(ws, L.gload);
  b.dxr = at<float>(ws, L.dxr);
  b.dpart = at<float>(ws, L.dpart);
  return hip_status(moe::launch_backward(a, b, stream));
}

moe_status_t moe_param_counts(const moe_config_t *cfg, int64_t *total, int64_t *active) {
  moe_status_t st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  if (!total || !active) return MOE_ERR_INVALID_ARGUMENT;
  const int64_t pe = (int64_t)(cfg->act == MOE_ACT_GELU ? 2 : 3) * cfg->d_model * cfg->d_hidden;
  const int64_t router = (int64_t)cfg->d_model * cfg->num_experts;
  *total = router + (cfg->num_experts + cfg->num_shared) * pe;
  *active = router + (cfg->top_k + cfg->num_shared) * pe;
  return MOE_OK;
}

moe_status_t moe_expert_capacity(int64_t num_tokens, int32_t top_k, int32_t num_experts,
                                 double factor, int32_t *capacity) {
  if (!capacity || num_tokens < 0 || top_k < 1 || num_experts < 1 || !(factor > 0.0))
    return MOE_ERR_INVALID_ARGUMENT;
  const double c = std::ceil(factor * (double)num_tokens * top_k / num_experts);
  if (!(c < 2147483647.0)) return MOE_ERR_UNSUPPORTED;
  *capacity = c < 1.0 ? 1 : (int32_t)c;
  return MOE_OK;
}

moe_status_t moe_load_stats(const int32_t *counts, const float *importance, int32_t E,
                            double *cv2_importance, double *cv2_load, double *load_balance) {
  if (!counts || E < 1 || !cv2_importance || !cv2_load || !load_balance)
    return MOE_ERR_INVALID_ARGUMENT;
  double sc = 0.0, si = 0.0;
  for (int e = 0; e < E; ++e) {
    sc += counts[e];
    if (importance) si += importance[e];
  }
  const double mc = sc / E, mi = si / E;
  double vc = 0.0, vi = 0.0, f2 = 0.0;
  for (int e = 0; e < E; ++e) {
    vc += (counts[e] - mc) * (counts[e] - mc);
    if (importance) vi += (importance[e] - mi) * (importance[e] - mi);
    if (sc != 0.0) f2 += (counts[e] / sc) * (counts[e] / sc);
  }
  *cv2_load = mc == 0.0 ? 0.0 : (vc / E) / (mc * mc);
  *cv2_importance = (!importance || mi == 0.0) ? 0.0 : (vi / E) / (mi * mi);
  *load_balance = sc == 0.0 ? 0.0 : E * f2;
  return MOE_OK;
}

}  // extern "C"
