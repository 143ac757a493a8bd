// backward.h - host-side interface of backward.hip (shared with api.cpp).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace moe {

int64_t bwd_padded_cols(int64_t T, int k, int E, int S);
hipError_t launch_fill_f32(float *p, int64_t n, hipStream_t s);

struct BwdBuffers {
  float *gimp, *ds;
  int32_t *poff, *colsrc;
  uint16_t *A, *H, *dyp, *dH, *dA, *dxp;
  uint16_t *dypT, *HT, *dAT, *xpT;
  // per-token m [T] and dense score gradients [T, E] (every gate); the
  // router's share of dx [T, d] (fp32; softmax-all and noisy gates)
  float *tm, *dS, *dxr;
  float *dpart;   // [splits, E, d] partial dW_g when the plan has several splits
  float *dU, *gload;   // noisy gate: noise-score gradients [T, E], Load term [E]
};

// Token splits of the dense router weight gradient dS^T x (its partial sums
// take splits * E * d floats when splits > 1).
void bwd_dense_plan(int64_t T, int E, int d, int *splits, int *kchunk);

struct BwdArgs {
  int T, k, E, S, d, h, swiglu, capacity;
  int bias_selects;   // the bias steers the selection only: it gets no gradient
  const uint16_t *x, *dy, *w_up, *w_down, *b_up, *w_up_s, *w_down_s;
  const float *w_gate;
  const int32_t *idx, *offsets, *pos;
  const float *topk_w, *importance;
  float w_imp;
  const uint16_t *x_perm, *y_perm;
  const uint16_t *hidden, *preact;   // from the training forward, or NULL
  const float *logits;   // the forward's router scores [T, E] (softmax-all gate), else NULL
  // noisy gate (clean != NULL): the forward's clean scores, Softplus scales,
  // draws, smooth Load and its loss weight; W_noise and its gradient
  const float *clean, *scale, *noise, *load, *w_noise;
  float w_load;
  float *dw_noise;
  uint16_t *dx;
  float *dw_gate, *db_gate;   // fp32, the router's dtype
  uint16_t *dw_up, *dw_down, *db_up, *db_down, *dw_up_s, *dw_down_s;   // bf16
};

hipError_t launch_backward(const BwdArgs &a, const BwdBuffers &b, hipStream_t s);

}  // namespace moe
