// backward.hip - the backward pass of the layer: the gradient of
// <dy, y> + w_imp * CV^2(Importance) with the top-k selection held fixed
// (the selection has no derivative; the router learns through the softmax
// weights: techfeed summary, "The hardest part: making the router
// trainable"; Importance and CV^2: Qiita summary, "Load-balancing losses").
//
// The grouped GEMMs of the backward pass run in gemm_bf16.hip (dH = dY W2,
// dX = dA W1 on the weights as stored, the weight gradients over each
// group's rows); this file holds the rest, all bf16 storage with fp32
// arithmetic:
//   gate     per token: dw_j = <dy, Y_j> (Y_j the expert's output row),
//            dY_j = w_j dy (the expert's output gradient, kept slots only),
//            ds_j = w_j (dw'_j - sum_i w_i dw'_i), dw'_j = dw_j + the
//            Importance term of expert i_j (softmax over the kept scores)
//   act      H = act(A) from the recomputed pre-activations A; dA = act'(A) dH
//   layout   group columns padded to 64 for the transposed copies, and the
//            grouped row behind every column
//   transpose activations [R, C] -> [C, Rp] (group columns, zero padding)
//   sums     per-group weighted row sums (bias and router gradients)
//   dx       dx = sum_j dX[pos_j] + dX_shared + sum_j ds_j W_g[i_j]
// Every sum runs in a fixed order: results are deterministic.
#include "common.h"
#include "backward.h"

#pragma clang fp contract(off)

namespace moe {

constexpr int kBwdThreads = 256;

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

// Sum over the workgroup in a fixed order (wave butterflies, then the waves
// in order); every thread gets the total.  red: kBwdThreads / 64 floats.
__device__ __forceinline__ float block_sum(float v, float *red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  const int wave = threadIdx.x / kWave;
  __syncthreads();
  if (threadIdx.x % kWave == 0) red[wave] = v;
  __syncthreads();
  float s = 0.0f;
#pragma unroll
  for (int w = 0; w < kBwdThreads / kWave; ++w) s += red[w];
  return s;
}

// Importance term of the gate gradient: d CV^2 / d I_e scaled by w_imp,
// CV^2 = V / m^2 with m the mean and V the population variance of I:
// g_e = w_imp * 2 (I_e - m - V / m) / (E m^2); zero when m = 0.
__global__ void bwd_importance_grad_kernel(const float *__restrict__ importance, int E,
                                           float w_imp, float *__restrict__ gimp) {
  __shared__ double mv[2];
  if (threadIdx.x == 0) {
    double m = 0.0;
    for (int e = 0; e < E; ++e) m += importance[e];
    m /= E;
    double v = 0.0;
    for (int e = 0; e < E; ++e) v += (importance[e] - m) * (importance[e] - m);
    mv[0] = m;
    mv[1] = v / E;
  }
  __syncthreads();
  const double m = mv[0], v = mv[1];
  for (int e = threadIdx.x; e < E; e += blockDim.x)
    gimp[e] = (m == 0.0 || w_imp == 0.0)
                  ? 0.0f
                  : (float)(w_imp * 2.0 * (importance[e] - m - v / m) / (E * m * m));
}

// One workgroup per token.  dyp: [T*k + S*T, d] expert output gradients
// (rows of dropped slots are not written); ds: [T, k] score gradients.
__global__ __launch_bounds__(kBwdThreads) void bwd_gate_kernel(
    const uint16_t *__restrict__ dy, const uint16_t *__restrict__ y_perm,
    const int32_t *__restrict__ pos, const int32_t *__restrict__ idx,
    const float *__restrict__ w, const float *__restrict__ gimp, int T, int k, int d, int E,
    int S, int rows, uint16_t *__restrict__ dyp, float *__restrict__ ds,
    float *__restrict__ tm) {
  __shared__ float red[kBwdThreads / kWave];
  __shared__ float dwp[kMaxExperts];
  const int t = blockIdx.x;
  const int nv = d / 8;   // 16-byte vectors per row
  const uint4 *dyr = reinterpret_cast<const uint4 *>(dy + (int64_t)t * d);
  for (int j = 0; j < k; ++j) {
    const int p = pos[(int64_t)t * k + j];
    const float wj = w[(int64_t)t * k + j];
    float part = 0.0f;
    if (p >= 0 && p < rows) {
      const uint4 *yr = reinterpret_cast<const uint4 *>(y_perm + (int64_t)p * d);
      uint4 *gr = reinterpret_cast<uint4 *>(dyp + (int64_t)p * d);
      for (int v = threadIdx.x; v < nv; v += kBwdThreads) {
        const uint4 a = dyr[v], b = yr[v];
        const uint32_t av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
        uint32_t o[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          part += bf16_lo(av[q]) * bf16_lo(bv[q]);
          part += bf16_hi(av[q]) * bf16_hi(bv[q]);
          o[q] = pack_bf16x2(wj * bf16_lo(av[q]), wj * bf16_hi(av[q]));
        }
        gr[v] = make_uint4(o[0], o[1], o[2], o[3]);
      }
    }
    const float dw = block_sum(part, red);
    if (threadIdx.x == 0) {
      const int e = idx[(int64_t)t * k + j];
      dwp[j] = dw + (gimp ? gimp[min(max(e, 0), E - 1)] : 0.0f);
    }
  }
  if (S) {
    uint4 *gr = reinterpret_cast<uint4 *>(dyp + ((int64_t)T * k + t) * d);
    for (int v = threadIdx.x; v < nv; v += kBwdThreads) gr[v] = dyr[v];
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float m = 0.0f;
    for (int j = 0; j < k; ++j) m += w[(int64_t)t * k + j] * dwp[j];
    for (int j = 0; j < k; ++j) {
      const float wj = w[(int64_t)t * k + j];
      ds[(int64_t)t * k + j] = wj * (dwp[j] - m);
    }
    if (tm) tm[t] = m;
  }
}

// H = act(A): GELU H = gelu(A) (A [R, h]); SwiGLU H[:, n] = silu(A[:, n]) *
// A[:, h + n] (A [R, 2h]).  8 columns per thread.
__global__ __launch_bounds__(kBwdThreads) void bwd_act_kernel(
    const uint16_t *__restrict__ A, int64_t R, int h, int swiglu, uint16_t *__restrict__ H) {
  const int nv = h / 8;
  const int na = swiglu ? 2 * h : h;
  for (int64_t i = blockIdx.x * (int64_t)kBwdThreads + threadIdx.x; i < R * nv;
       i += (int64_t)gridDim.x * kBwdThreads) {
    const int64_t r = i / nv;
    const int c = (int)(i % nv) * 8;
    const uint4 g4 = *reinterpret_cast<const uint4 *>(A + r * na + c);
    const uint32_t gv[4] = {g4.x, g4.y, g4.z, g4.w};
    uint32_t o[4];
    if (swiglu) {
      const uint4 u4 = *reinterpret_cast<const uint4 *>(A + r * na + h + c);
      const uint32_t uv[4] = {u4.x, u4.y, u4.z, u4.w};
#pragma unroll
      for (int q = 0; q < 4; ++q)
        o[q] = pack_bf16x2(silu_f32(bf16_lo(gv[q])) * bf16_lo(uv[q]),
                           silu_f32(bf16_hi(gv[q])) * bf16_hi(uv[q]));
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        o[q] = pack_bf16x2(gelu_f32(bf16_lo(gv[q])), gelu_f32(bf16_hi(gv[q])));
    }
    *reinterpret_cast<uint4 *>(H + r * h + c) = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

// dA = act'(A) dH.  GELU: dA = dH (Phi(a) + a phi(a)).  SwiGLU, h = silu(g) u:
// dg = dH u sigma(g) (1 + g (1 - sigma(g))), du = dH silu(g).
__device__ __forceinline__ float gelu_grad(float a) {
  const float cdf = 0.5f * (1.0f + erff(a * 0.70710678118654752f));
  const float pdf = 0.39894228040143268f * expf(-0.5f * a * a);
  return cdf + a * pdf;
}

__global__ __launch_bounds__(kBwdThreads) void bwd_act_grad_kernel(
    const uint16_t *__restrict__ A, const uint16_t *__restrict__ dH, int64_t R, int h,
    int swiglu, uint16_t *__restrict__ dA) {
  const int nv = h / 8;
  const int na = swiglu ? 2 * h : h;
  for (int64_t i = blockIdx.x * (int64_t)kBwdThreads + threadIdx.x; i < R * nv;
       i += (int64_t)gridDim.x * kBwdThreads) {
    const int64_t r = i / nv;
    const int c = (int)(i % nv) * 8;
    const uint4 g4 = *reinterpret_cast<const uint4 *>(A + r * na + c);
    const uint4 d4 = *reinterpret_cast<const uint4 *>(dH + r * h + c);
    const uint32_t gv[4] = {g4.x, g4.y, g4.z, g4.w}, dv[4] = {d4.x, d4.y, d4.z, d4.w};
    uint32_t og[4];
    if (swiglu) {
      const uint4 u4 = *reinterpret_cast<const uint4 *>(A + r * na + h + c);
      const uint32_t uv[4] = {u4.x, u4.y, u4.z, u4.w};
      uint32_t ou[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float dg[2], du[2];
        const float gs[2] = {bf16_lo(gv[q]), bf16_hi(gv[q])};
        const float us[2] = {bf16_lo(uv[q]), bf16_hi(uv[q])};
        const float hs[2] = {bf16_lo(dv[q]), bf16_hi(dv[q])};
#pragma unroll
        for (int z = 0; z < 2; ++z) {
          const float sg = 1.0f / (1.0f + expf(-gs[z]));
          dg[z] = hs[z] * us[z] * sg * (1.0f + gs[z] * (1.0f - sg));
          du[z] = hs[z] * gs[z] * sg;
        }
        og[q] = pack_bf16x2(dg[0], dg[1]);
        ou[q] = pack_bf16x2(du[0], du[1]);
      }
      *reinterpret_cast<uint4 *>(dA + r * na + h + c) = make_uint4(ou[0], ou[1], ou[2], ou[3]);
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        og[q] = pack_bf16x2(bf16_lo(dv[q]) * gelu_grad(bf16_lo(gv[q])),
                            bf16_hi(dv[q]) * gelu_grad(bf16_hi(gv[q])));
    }
    *reinterpret_cast<uint4 *>(dA + r * na + c) = make_uint4(og[0], og[1], og[2], og[3]);
  }
}

// Group g's rows: routed groups [offsets[g], offsets[g+1]) (clamped), the
// shared group (g == E) rows [T*k, T*k + T).  poff: exclusive scan of the
// row counts rounded up to 64.  One workgroup of kMaxExperts + 1 <= 2 *
// 256 groups: thread t owns groups 2t and 2t + 1.
__global__ __launch_bounds__(kBwdThreads) void bwd_layout_kernel(
    const int32_t *__restrict__ offsets, int E, int S, int T, int routed,
    int32_t *__restrict__ poff) {
  __shared__ int sc[kBwdThreads];
  const int G = E + S;
  const int tid = threadIdx.x;
  int c[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int g = 2 * tid + q;
    int n = 0;
    if (g < E) {
      const int r0 = min(max(offsets[g], 0), routed);
      const int r1 = min(max(offsets[g + 1], r0), routed);
      n = r1 - r0;
    } else if (g < G) {
      n = T;
    }
    c[q] = (n + 63) / 64 * 64;
  }
  sc[tid] = c[0] + c[1];
  __syncthreads();
  for (int off = 1; off < kBwdThreads; off <<= 1) {
    const int v = tid >= off ? sc[tid - off] : 0;
    __syncthreads();
    sc[tid] += v;
    __syncthreads();
  }
  const int ex = sc[tid] - c[0] - c[1];
  if (2 * tid <= G) poff[2 * tid] = ex;
  if (2 * tid + 1 <= G) poff[2 * tid + 1] = ex + c[0];
}

// colsrc[j]: the grouped row behind padded column j, or -1 (padding).
__global__ __launch_bounds__(kBwdThreads) void bwd_colsrc_kernel(
    const int32_t *__restrict__ offsets, const int32_t *__restrict__ poff, int E, int S,
    int T, int routed, int Rp, int32_t *__restrict__ colsrc) {
  const int G = E + S;
  for (int j = blockIdx.x * kBwdThreads + threadIdx.x; j < Rp; j += gridDim.x * kBwdThreads) {
    int v = -1;
    if (j < poff[G]) {
      int lo = 0, hi = G - 1;   // last group with poff[g] <= j
      while (lo < hi) {
        const int mid = (lo + hi + 1) / 2;
        if (poff[mid] <= j) lo = mid; else hi = mid - 1;
      }
      int r0, n;
      if (lo < E) {
        r0 = min(max(offsets[lo], 0), routed);
        n = min(max(offsets[lo + 1], r0), routed) - r0;
      } else {
        r0 = routed;
        n = T;
      }
      if (j - poff[lo] < n) v = r0 + (j - poff[lo]);
    }
    colsrc[j] = v;
  }
}

// dst[c][j] = row colsrc[j] of the source (routed rows from src, rows from
// `routed` on from src_shared), column c; 0 on padding.  64 x 64 tiles
// through LDS, 16-byte global accesses on both sides.  C % 64 == 0, Rp % 64
// == 0.
__global__ __launch_bounds__(kBwdThreads) void bwd_transpose_cols_kernel(
    const uint16_t *__restrict__ src, const uint16_t *__restrict__ src_shared, int routed,
    int C, const int32_t *__restrict__ colsrc, int Rp, uint16_t *__restrict__ dst) {
  __shared__ uint16_t tile[64][64 + 2];
  const int j0 = blockIdx.x * 64;
  const int c0 = blockIdx.y * 64;
  const int tid = threadIdx.x;
  // load: 64 source rows x 8 vectors of 8 columns
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int q = tid + i * kBwdThreads;
    const int jj = q / 8, v = q % 8;
    const int r = colsrc[j0 + jj];
    uint4 val = make_uint4(0, 0, 0, 0);
    if (r >= 0) {
      const uint16_t *row = r < routed ? src + (int64_t)r * C
                                       : src_shared + (int64_t)(r - routed) * C;
      val = *reinterpret_cast<const uint4 *>(row + c0 + 8 * v);
    }
    const uint32_t w4[4] = {val.x, val.y, val.z, val.w};
#pragma unroll
    for (int z = 0; z < 4; ++z) {
      tile[jj][8 * v + 2 * z] = (uint16_t)(w4[z] & 0xffffu);
      tile[jj][8 * v + 2 * z + 1] = (uint16_t)(w4[z] >> 16);
    }
  }
  __syncthreads();
  // store: 64 destination rows (c) x 8 vectors of 8 columns (j)
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int q = tid + i * kBwdThreads;
    const int cc = q / 8, v = q % 8;
    uint32_t w4[4];
#pragma unroll
    for (int z = 0; z < 4; ++z)
      w4[z] = (uint32_t)tile[8 * v + 2 * z][cc] | ((uint32_t)tile[8 * v + 2 * z + 1][cc] << 16);
    *reinterpret_cast<uint4 *>(dst + (int64_t)(c0 + cc) * Rp + j0 + 8 * v) =
        make_uint4(w4[0], w4[1], w4[2], w4[3]);
  }
}

// out[g][c] = sum over group g's columns j of at[c][j] (bf16 bias
// gradients), for groups g < G; one wavefront per (g, c): lanes take
// columns j = lane, lane + 64, ... in order, then a fixed butterfly.
__global__ __launch_bounds__(kWave) void bwd_rowsum_kernel(
    const uint16_t *__restrict__ at, int C, int Rp, const int32_t *__restrict__ poff,
    uint16_t *__restrict__ out) {
  const int c = blockIdx.x;
  const int g = blockIdx.y;
  const int lane = threadIdx.x;
  const int j0 = poff[g], j1 = poff[g + 1];
  const uint16_t *row = at + (int64_t)c * Rp;
  float s = 0.0f;
  for (int j = j0 + lane; j < j1; j += kWave) s += __uint_as_float((uint32_t)row[j] << 16);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
  if (lane == 0) out[(int64_t)g * C + c] = (uint16_t)(pack_bf16x2(s, 0.0f) & 0xffffu);
}

// dx[t] = sum_j dX[pos_j] + dX[T*k + t] (shared) + sum_j ds_j W_g[i_j], fp32
// accumulation in that order, one rounding to bf16.  One workgroup per
// token, 4 columns per thread.
__global__ __launch_bounds__(kBwdThreads) void bwd_dx_kernel(
    const uint16_t *__restrict__ dxp, const int32_t *__restrict__ pos,
    const float *__restrict__ ds, const int32_t *__restrict__ idx,
    const float *__restrict__ wg, const float *__restrict__ dxr, int T, int k, int d, int E,
    int S, int rows, uint16_t *__restrict__ dx) {
  const int t = blockIdx.x;
  for (int c = 4 * threadIdx.x; c < d; c += 4 * kBwdThreads) {
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < k; ++j) {
      const int p = pos[(int64_t)t * k + j];
      if (p < 0 || p >= rows) continue;
      const uint2 v = *reinterpret_cast<const uint2 *>(dxp + (int64_t)p * d + c);
      acc[0] += bf16_lo(v.x);
      acc[1] += bf16_hi(v.x);
      acc[2] += bf16_lo(v.y);
      acc[3] += bf16_hi(v.y);
    }
    if (S) {
      const uint2 v = *reinterpret_cast<const uint2 *>(dxp + ((int64_t)T * k + t) * d + c);
      acc[0] += bf16_lo(v.x);
      acc[1] += bf16_hi(v.x);
      acc[2] += bf16_lo(v.y);
      acc[3] += bf16_hi(v.y);
    }
    if (dxr) {   // dense router term (softmax-all and noisy gates)
      const float4 r = *reinterpret_cast<const float4 *>(dxr + (int64_t)t * d + c);
      acc[0] += r.x;
      acc[1] += r.y;
      acc[2] += r.z;
      acc[3] += r.w;
    } else {
      for (int j = 0; j < k; ++j) {
        const int e = min(max(idx[(int64_t)t * k + j], 0), E - 1);
        const float sj = ds[(int64_t)t * k + j];
        const float4 wv = *reinterpret_cast<const float4 *>(wg + (int64_t)e * d + c);
        acc[0] += sj * wv.x;
        acc[1] += sj * wv.y;
        acc[2] += sj * wv.z;
        acc[3] += sj * wv.w;
      }
    }
    uint2 o;
    o.x = pack_bf16x2(acc[0], acc[1]);
    o.y = pack_bf16x2(acc[2], acc[3]);
    *reinterpret_cast<uint2 *>(dx + (int64_t)t * d + c) = o;
  }
}

// Dense score gradients dS [T, E], one wavefront per token.  A kept expert
// takes the ds of the gate kernel.  Softmax-all gate (logits given): the gate
// values are w_j = p_{i_j} with p the softmax of all E scores, so every
// score has a gradient: ds_e = p_e (dw'_e [e kept] - m) with m = sum_j w_j
// dw'_j, which for a kept expert is that ds.  Otherwise (logits NULL) an
// unkept score has none: zero.
__global__ __launch_bounds__(kWave) void bwd_dense_ds_kernel(
    const float *__restrict__ logits, const int32_t *__restrict__ idx,
    const float *__restrict__ ds, const float *__restrict__ tm, int T, int E, int k,
    float *__restrict__ dS) {
  const int t = blockIdx.x;
  const int lane = threadIdx.x;
  const float *s = logits ? logits + (int64_t)t * E : nullptr;
  float mx = -INFINITY, z = 0.0f, m = 0.0f;
  if (s) {
    for (int e = lane; e < E; e += kWave) mx = fmaxf(mx, s[e]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    for (int e = lane; e < E; e += kWave) z += expf(s[e] - mx);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) z += __shfl_xor(z, off);
    m = tm[t];
  }
  const int32_t *it = idx + (int64_t)t * k;
  float *row = dS + (int64_t)t * E;
  for (int e = lane; e < E; e += kWave) {
    int j = 0;
    while (j < k && it[j] != e) ++j;
    row[e] = j < k ? ds[(int64_t)t * k + j] : (s ? -(expf(s[e] - mx) / z) * m : 0.0f);
  }
}

// Noisy gate (H = s + n * Softplus(u), u = x W_noise^T; the kept weights are
// the softmax of the kept H) with the smooth Load P(x, i) = Phi(z_i), z_i =
// (s_i - H_{j(i)}) / Softplus_i, j(i) the k-th ranked entry of H when i is
// not kept and the (k+1)-th when it is.  One wavefront per token writes the
// dense gradients of the clean scores s and of the noise scores u:
//   a_i    = gload_i phi(z_i) / Softplus_i       (gload: d w_load CV^2 / d Load)
//   dH_i   = ds_j [i kept as slot j] - [i = k-th] sum_{unkept} a - [i = (k+1)-th]
//            sum_{kept} a
//   dS_i   = dH_i + a_i
//   dU_i   = sigmoid(u_i) (n_i dH_i - a_i z_i),  sigmoid(u) = 1 - exp(-Softplus(u))
// H is recomputed with the forward's one fused multiply-add, so the ranks
// are the forward's.
__global__ __launch_bounds__(kWave) void bwd_noisy_ds_kernel(
    const float *__restrict__ clean, const float *__restrict__ scale,
    const float *__restrict__ noise, const int32_t *__restrict__ idx,
    const float *__restrict__ ds, const float *__restrict__ gload, int E, int k,
    float *__restrict__ dS, float *__restrict__ dU) {
  constexpr int Q = kMaxExperts / kWave;
  const int t = blockIdx.x;
  const int lane = threadIdx.x;
  const int64_t row = (int64_t)t * E;
  const int32_t *it = idx + (int64_t)t * k;
  float sv[Q], sg[Q], nv[Q], hv[Q], dh[Q];
  int slot[Q];
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const int e = lane + kWave * q;
    const bool ok = e < E;
    sv[q] = ok ? clean[row + e] : 0.0f;
    sg[q] = ok ? scale[row + e] : 0.0f;
    nv[q] = ok ? noise[row + e] : 0.0f;
    hv[q] = fmaf(nv[q], sg[q], sv[q]);
    int j = -1;
    for (int i = 0; i < k && ok; ++i)
      if (it[i] == e) j = i;
    slot[q] = j;
    dh[q] = j >= 0 ? ds[(int64_t)t * k + j] : 0.0f;
  }
  float a[Q], z[Q];
#pragma unroll
  for (int q = 0; q < Q; ++q) a[q] = z[q] = 0.0f;
  int jk = -1, jk1 = -1;
  if (gload && k < E) {
    jk = min(max(it[k - 1], 0), E - 1);   // clamped: a corrupt index stays in the row
    // the (k+1)-th: the best entry outside the kept k (H descending, index
    // ascending), a wavefront arg-max
    bool ba = false;
    float bh = 0.0f;
    int be = 0x7fffffff;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int e = lane + kWave * q;
      if (e < E && slot[q] < 0 && (!ba || hv[q] > bh || (hv[q] == bh && e < be))) {
        ba = true;
        bh = hv[q];
        be = e;
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const bool oa = __shfl_xor((int)ba, off) != 0;
      const float oh = __shfl_xor(bh, off);
      const int oe = __shfl_xor(be, off);
      if (oa && (!ba || oh > bh || (oh == bh && oe < be))) {
        ba = true;
        bh = oh;
        be = oe;
      }
    }
    // none only if the kept slots name every expert (a corrupt selection):
    // then no entry takes the kept experts' term, and the load stays in range
    jk1 = ba ? be : -1;
    const int j1 = ba ? be : jk;
    const float hk = fmaf(noise[row + jk], scale[row + jk], clean[row + jk]);
    const float hk1 = fmaf(noise[row + j1], scale[row + j1], clean[row + j1]);
    constexpr float kInvSqrt2Pi = 0.3989422804014327f;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int e = lane + kWave * q;
      if (e < E && sg[q] > 0.0f) {
        z[q] = (sv[q] - (slot[q] >= 0 ? hk1 : hk)) / sg[q];
        a[q] = gload[e] * kInvSqrt2Pi * expf(-0.5f * z[q] * z[q]) / sg[q];
      }
    }
  }
  float ak = 0.0f, au = 0.0f;   // sums of a over the kept and the other entries
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    if (slot[q] >= 0)
      ak += a[q];
    else
      au += a[q];
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    ak += __shfl_xor(ak, off);
    au += __shfl_xor(au, off);
  }
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const int e = lane + kWave * q;
    if (e >= E) continue;
    float dht = dh[q];
    if (e == jk) dht -= au;
    if (e == jk1) dht -= ak;
    dS[row + e] = dht + a[q];
    const float sigm = -expm1f(-sg[q]);
    dU[row + e] = sigm * (nv[q] * dht - a[q] * z[q]);
  }
}

// Dense fp32 products of the router gradients on the
// fp32 matrix cores (v_mfma_f32_16x16x4_f32: lane l supplies A[l%16][l/16]
// and B[l/16][l%16], and holds D[4(l/16)+r][l%16] in r = 0..3):
//   C_z[m][n] = sum over k in split z of A(m, k) B[k][n]
// with B [K][N] row-major (bf16 or fp32) and A [K][M] (AT) or [M][K].
// Workgroup of 4 wavefronts (WM x WN), each a (16 MT) x (16 NT) block of
// C; k in stages of 16 through LDS (rows padded by 16 floats so that the 4
// k-rows of one MFMA operand fall in different banks), the next stage
// loaded into registers while the current one is multiplied.
template <bool AT>
__device__ inline void dense_ld_a(const float *__restrict__ A, int M, int K, int m, int k,
                                  float (&v)[4]) {
  // AT: 4 consecutive m of row k; else 4 consecutive k of row m
  const int64_t off = AT ? (int64_t)k * M + m : (int64_t)m * K + k;
  const int n_ok = AT ? (k < K ? min(4, M - m) : 0) : (m < M ? min(4, K - k) : 0);
  if (n_ok == 4 && (AT ? M % 4 == 0 : K % 4 == 0)) {
    const float4 q = *reinterpret_cast<const float4 *>(A + off);
    v[0] = q.x, v[1] = q.y, v[2] = q.z, v[3] = q.w;
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = j < n_ok ? A[off + j] : 0.0f;
  }
}

__device__ inline void dense_ld_b(const float *__restrict__ B, int64_t off, bool ok,
                                  float (&v)[4]) {
  const float4 q = ok ? *reinterpret_cast<const float4 *>(B + off) : make_float4(0, 0, 0, 0);
  v[0] = q.x, v[1] = q.y, v[2] = q.z, v[3] = q.w;
}

__device__ inline void dense_ld_b(const uint16_t *__restrict__ B, int64_t off, bool ok,
                                  float (&v)[4]) {
  const uint2 q = ok ? *reinterpret_cast<const uint2 *>(B + off) : make_uint2(0, 0);
  v[0] = __uint_as_float(q.x << 16), v[1] = __uint_as_float(q.x & 0xffff0000u);
  v[2] = __uint_as_float(q.y << 16), v[3] = __uint_as_float(q.y & 0xffff0000u);
}

template <int WM, int WN, int MT, int NT, bool AT, typename BT>
__global__ __launch_bounds__(256) void bwd_dense_gemm_kernel(
    const float *__restrict__ A, const BT *__restrict__ B, int M, int N, int K, int kchunk,
    int accumulate, float *__restrict__ C) {
  static_assert(WM * WN == 4, "four wavefronts");
  constexpr int BM = WM * MT * 16, BN = WN * NT * 16, BK = 16;
  constexpr int PA = BM + 16, PB = BN + 16;
  constexpr int CA = BK * BM / 4, CB = BK * BN / 4;   // float4 chunks per stage
  constexpr int NA = (CA + 255) / 256, NB = (CB + 255) / 256;
  __shared__ float As[BK][PA];
  __shared__ float Bs[BK][PB];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const int kb = blockIdx.z * kchunk, ke = min(K, kb + kchunk);
  float ra[NA][4], rb[NB][4];
  auto load = [&](int k0) {
#pragma unroll
    for (int q = 0; q < NA; ++q) {
      const int i = tid + 256 * q;
      if (i >= CA) break;
      const int mm = AT ? (i % (BM / 4)) * 4 : i / (BK / 4);
      const int kk = AT ? i / (BM / 4) : (i % (BK / 4)) * 4;
      if (AT) {
        dense_ld_a<true>(A, M, k0 + kk < ke ? K : 0, m0 + mm, k0 + kk, ra[q]);
      } else {
        // the k-range of this split bounds the row
        dense_ld_a<false>(A, M, K, m0 + mm, k0 + kk, ra[q]);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (k0 + kk + j >= ke) ra[q][j] = 0.0f;
      }
    }
#pragma unroll
    for (int q = 0; q < NB; ++q) {
      const int i = tid + 256 * q;
      if (i >= CB) break;
      const int kk = i / (BN / 4), nn = (i % (BN / 4)) * 4;
      const int k = k0 + kk, n = n0 + nn;
      dense_ld_b(B, (int64_t)k * N + n, k < ke && n < N, rb[q]);
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int q = 0; q < NA; ++q) {
      const int i = tid + 256 * q;
      if (i >= CA) break;
      if (AT) {
        const int kk = i / (BM / 4), mm = (i % (BM / 4)) * 4;
#pragma unroll
        for (int j = 0; j < 4; ++j) As[kk][mm + j] = ra[q][j];
      } else {
        const int mm = i / (BK / 4), kk = (i % (BK / 4)) * 4;
#pragma unroll
        for (int j = 0; j < 4; ++j) As[kk + j][mm] = ra[q][j];
      }
    }
#pragma unroll
    for (int q = 0; q < NB; ++q) {
      const int i = tid + 256 * q;
      if (i >= CB) break;
      const int kk = i / (BN / 4), nn = (i % (BN / 4)) * 4;
#pragma unroll
      for (int j = 0; j < 4; ++j) Bs[kk][nn + j] = rb[q][j];
    }
  };
  f32x4_t acc[MT][NT];
#pragma unroll
  for (int a = 0; a < MT; ++a)
#pragma unroll
    for (int b = 0; b < NT; ++b) acc[a][b] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  if (kb < ke) load(kb);
  for (int k0 = kb; k0 < ke; k0 += BK) {
    __syncthreads();
    store();
    __syncthreads();
    if (k0 + BK < ke) load(k0 + BK);
    const int r = lane >> 4, c = lane & 15;
#pragma unroll
    for (int ks = 0; ks < BK; ks += 4) {
      float av[MT], bv[NT];
#pragma unroll
      for (int a = 0; a < MT; ++a) av[a] = As[ks + r][(wm * MT + a) * 16 + c];
#pragma unroll
      for (int b = 0; b < NT; ++b) bv[b] = Bs[ks + r][(wn * NT + b) * 16 + c];
#pragma unroll
      for (int a = 0; a < MT; ++a)
#pragma unroll
        for (int b = 0; b < NT; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[a], bv[b], acc[a][b], 0, 0, 0);
    }
  }
  float *Cz = C + (int64_t)blockIdx.z * M * N;
  const int r = lane >> 4, c = lane & 15;
#pragma unroll
  for (int a = 0; a < MT; ++a)
#pragma unroll
    for (int b = 0; b < NT; ++b) {
      const int n = n0 + (wn * NT + b) * 16 + c;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int m = m0 + (wm * MT + a) * 16 + 4 * r + q;
        if (m < M && n < N) {
          float *c = Cz + (int64_t)m * N + n;
          *c = accumulate ? *c + acc[a][b][q] : acc[a][b][q];
        }
      }
    }
}

// out[i] = sum over the splits z (ascending) of part[z][i], float4 lanes.
__global__ void bwd_split_sum_kernel(const float *__restrict__ part, int splits, int64_t n4,
                                     float *__restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n4) return;
  const float4 *p = reinterpret_cast<const float4 *>(part) + i;
  float4 s = p[0];
  for (int z = 1; z < splits; ++z) {
    const float4 v = p[(int64_t)z * n4];
    s.x += v.x, s.y += v.y, s.z += v.z, s.w += v.w;
  }
  reinterpret_cast<float4 *>(out)[i] = s;
}

// db[e] = sum_t dS[t][e]: one wavefront per expert, lanes take t = lane,
// lane + 64, ... in order, then a fixed butterfly.
__global__ __launch_bounds__(kWave) void bwd_dense_bias_kernel(
    const float *__restrict__ dS, int T, int E, float *__restrict__ db) {
  const int e = blockIdx.x;
  float s = 0.0f;
  for (int t = threadIdx.x; t < T; t += kWave) s += dS[(int64_t)t * E + e];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
  if (threadIdx.x == 0) db[e] = s;
}

__global__ void bwd_fill_f32_kernel(float *p, int64_t n, float v) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

// ------------------------------------------------------------------ host --

hipError_t launch_grouped_linear_bf16(const int32_t *offsets, int E, int S, int T, int k,
                                      int K, int n_out, const void *a_routed,
                                      const void *a_shared, const void *w,
                                      const void *w_shared, const void *bias, void *c,
                                      bool w_kn, hipStream_t s);
hipError_t launch_wgrad_bf16(const int32_t *poff, int G, int Rp, int M, int N, const void *at,
                             const void *bt, void *out, void *out_last, hipStream_t s);

static unsigned grid_for(int64_t work, int64_t per_block) {
  int64_t b = (work + per_block - 1) / per_block;
  if (b > 4096) b = 4096;
  return (unsigned)(b < 1 ? 1 : b);
}

hipError_t launch_fill_f32(float *p, int64_t n, hipStream_t s) {
  if (!p || n <= 0) return hipSuccess;
  bwd_fill_f32_kernel<<<grid_for(n, 256), 256, 0, s>>>(p, n, 0.0f);
  return hipGetLastError();
}

// Columns of the transposed copies: every group padded to 64, rounded to an
// odd multiple of 64 so that the row stride is an odd number of 128-byte
// lines (rows then spread over the cache sets instead of aliasing).
int64_t bwd_padded_cols(int64_t T, int k, int E, int S) {
  const int64_t R = T * k + (int64_t)S * T;
  const int64_t n64 = (R + 64 * (int64_t)(E + S) + 63) / 64;
  return 64 * (n64 | 1);
}

// Token splits of the dense router weight gradient: enough workgroups to
// fill the chip (about 1024), at least 128 tokens a split.
void bwd_dense_plan(int64_t T, int E, int d, int *splits, int *kchunk) {
  const int64_t tiles = E <= 32 ? (int64_t)((E + 15) / 16) * ((d + 255) / 256)
                                : (int64_t)((E + 127) / 128) * ((d + 127) / 128);
  int64_t z = std::max<int64_t>(1, std::min<int64_t>((1024 + tiles - 1) / tiles,
                                                     (T + 127) / 128));
  int64_t kc = ((T + z - 1) / z + 15) / 16 * 16;
  *kchunk = (int)std::max<int64_t>(kc, 16);
  *splits = (int)std::max<int64_t>(1, (T + *kchunk - 1) / *kchunk);
}

hipError_t launch_backward(const BwdArgs &a, const BwdBuffers &b, hipStream_t s) {
  const int T = a.T, k = a.k, E = a.E, S = a.S, d = a.d, h = a.h;
  const int G = E + S;
  const int routed = T * k;
  const int R = routed + S * T;
  const int nup = a.swiglu ? 2 * h : h;
  const int Rp = (int)bwd_padded_cols(T, k, E, S);
  hipError_t err;
#define MOE_TRY(x)                         \
  do {                                     \
    if ((err = (x)) != hipSuccess) return err; \
  } while (0)

  // gate: Importance term, expert output gradients, score gradients
  const float *gimp = nullptr;
  if (a.importance && a.w_imp != 0.0f) {
    bwd_importance_grad_kernel<<<1, kBwdThreads, 0, s>>>(a.importance, E, a.w_imp, b.gimp);
    gimp = b.gimp;
  }
  // The score gradients as a dense [T, E] matrix for every gate (zero where
  // a score has none), so that the router's weight gradient is one GEMM
  // dS^T X whatever the selection and the drops (a dropped slot still has a
  // score gradient: its gate shapes the kept softmax and Importance).  The
  // softmax-all and noisy gates give every score a gradient, and then the
  // router's share of dx is dense too (the noisy gate's noise scores also).
  const bool noisy = a.clean != nullptr;
  const bool dense = a.logits != nullptr || noisy;
  bwd_gate_kernel<<<T, kBwdThreads, 0, s>>>(a.dy, a.y_perm, a.pos, a.idx, a.topk_w, gimp, T,
                                            k, d, E, S, R, b.dyp, b.ds, a.logits ? b.tm : nullptr);
  MOE_TRY(hipGetLastError());
  if (noisy) {
    const float *gload = nullptr;
    if (a.load && a.w_load != 0.0f) {
      bwd_importance_grad_kernel<<<1, kBwdThreads, 0, s>>>(a.load, E, a.w_load, b.gload);
      gload = b.gload;
    }
    bwd_noisy_ds_kernel<<<T, kWave, 0, s>>>(a.clean, a.scale, a.noise, a.idx, b.ds, gload, E, k,
                                            b.dS, b.dU);
  } else {
    bwd_dense_ds_kernel<<<T, kWave, 0, s>>>(a.logits, a.idx, b.ds, b.tm, T, E, k, b.dS);
  }
  MOE_TRY(hipGetLastError());
  if (dense) {
    // the router's share of dx: dS [T, E] times W_g [E, d] (+ dU W_noise);
    // otherwise the gate kernel's k score gradients per token serve
    const dim3 grid((d + 127) / 128, (T + 127) / 128, 1);
    bwd_dense_gemm_kernel<2, 2, 4, 4, false, float>
        <<<grid, 256, 0, s>>>(b.dS, a.w_gate, T, d, E, E, 0, b.dxr);
    if (noisy)
      bwd_dense_gemm_kernel<2, 2, 4, 4, false, float>
          <<<grid, 256, 0, s>>>(b.dU, a.w_noise, T, d, E, E, 1, b.dxr);
    MOE_TRY(hipGetLastError());
  }

  // padded group columns
  bwd_layout_kernel<<<1, kBwdThreads, 0, s>>>(a.offsets, E, S, T, routed, b.poff);
  bwd_colsrc_kernel<<<grid_for(Rp, kBwdThreads), kBwdThreads, 0, s>>>(a.offsets, b.poff, E, S, T,
                                                                       routed, Rp, b.colsrc);
  MOE_TRY(hipGetLastError());

  // pre-activations (the training forward's, else recomputed), activations,
  // then the chain back to dX
  const uint16_t *A = a.preact ? a.preact : b.A;
  const uint16_t *H = a.hidden ? a.hidden : b.H;
  if (!a.preact)
    MOE_TRY(launch_grouped_linear_bf16(a.offsets, E, S, T, k, d, nup, a.x_perm, a.x, a.w_up,
                                       a.w_up_s, a.swiglu ? nullptr : a.b_up, b.A, false, s));
  if (!a.hidden)
    bwd_act_kernel<<<grid_for((int64_t)R * (h / 8), kBwdThreads), kBwdThreads, 0, s>>>(
        A, R, h, a.swiglu, b.H);
  // dH = dY W2 and dX = dA W1 read W2 [d][h] and W1 [nup][d] as stored
  // (k-row weights), no transposed copies
  MOE_TRY(launch_grouped_linear_bf16(a.offsets, E, S, T, k, d, h, b.dyp,
                                     b.dyp + (int64_t)routed * d, a.w_down, a.w_down_s, nullptr,
                                     b.dH, true, s));
  bwd_act_grad_kernel<<<grid_for((int64_t)R * (h / 8), kBwdThreads), kBwdThreads, 0, s>>>(
      A, b.dH, R, h, a.swiglu, b.dA);
  MOE_TRY(launch_grouped_linear_bf16(a.offsets, E, S, T, k, nup, d, b.dA,
                                     b.dA + (int64_t)routed * nup, a.w_up, a.w_up_s, nullptr,
                                     b.dxp, true, s));
  bwd_dx_kernel<<<T, kBwdThreads, 0, s>>>(b.dxp, a.pos, b.ds, a.idx, a.w_gate,
                                         dense ? b.dxr : nullptr, T, k, d, E, S, R, a.dx);
  MOE_TRY(hipGetLastError());

  // weight gradients over each group's rows
  bwd_transpose_cols_kernel<<<dim3(Rp / 64, d / 64), kBwdThreads, 0, s>>>(
      b.dyp, b.dyp + (int64_t)routed * d, routed, d, b.colsrc, Rp, b.dypT);
  bwd_transpose_cols_kernel<<<dim3(Rp / 64, h / 64), kBwdThreads, 0, s>>>(
      H, H + (int64_t)routed * h, routed, h, b.colsrc, Rp, b.HT);
  bwd_transpose_cols_kernel<<<dim3(Rp / 64, nup / 64), kBwdThreads, 0, s>>>(
      b.dA, b.dA + (int64_t)routed * nup, routed, nup, b.colsrc, Rp, b.dAT);
  bwd_transpose_cols_kernel<<<dim3(Rp / 64, d / 64), kBwdThreads, 0, s>>>(
      a.x_perm, a.x, routed, d, b.colsrc, Rp, b.xpT);
  MOE_TRY(hipGetLastError());
  MOE_TRY(launch_wgrad_bf16(b.poff, G, Rp, d, h, b.dypT, b.HT, a.dw_down,
                            S ? a.dw_down_s : nullptr, s));
  MOE_TRY(launch_wgrad_bf16(b.poff, G, Rp, nup, d, b.dAT, b.xpT, a.dw_up,
                            S ? a.dw_up_s : nullptr, s));
  if (a.db_down)
    bwd_rowsum_kernel<<<dim3(d, E), kWave, 0, s>>>(b.dypT, d, Rp, b.poff, a.db_down);
  if (a.db_up)
    bwd_rowsum_kernel<<<dim3(h, E), kWave, 0, s>>>(b.dAT, h, Rp, b.poff, a.db_up);
  // router: dW = dS^T X over token splits, then the splits summed in order
  // (and dW_noise = dU^T X for the noisy gate); db = the column sums of dS,
  // zero under the bias-selects gate (the bias there only steers selection)
  int splits, kchunk;
  bwd_dense_plan(T, E, d, &splits, &kchunk);
  auto wgrad = [&](const float *dsc, float *out) {
    float *dst = splits > 1 ? b.dpart : out;
    if (E <= 32)
      bwd_dense_gemm_kernel<1, 4, 1, 4, true, uint16_t>
          <<<dim3((d + 255) / 256, (E + 15) / 16, splits), 256, 0, s>>>(dsc, a.x, E, d, T,
                                                                        kchunk, 0, dst);
    else
      bwd_dense_gemm_kernel<2, 2, 4, 4, true, uint16_t>
          <<<dim3((d + 127) / 128, (E + 127) / 128, splits), 256, 0, s>>>(dsc, a.x, E, d, T,
                                                                          kchunk, 0, dst);
    if (splits > 1) {
      const int64_t n4 = (int64_t)E * d / 4;
      bwd_split_sum_kernel<<<grid_for(n4, 256), 256, 0, s>>>(b.dpart, splits, n4, out);
    }
  };
  wgrad(b.dS, a.dw_gate);
  if (noisy) wgrad(b.dU, a.dw_noise);
  if (a.db_gate) {
    if (a.bias_selects)
      MOE_TRY(launch_fill_f32(a.db_gate, E, s));
    else
      bwd_dense_bias_kernel<<<E, kWave, 0, s>>>(b.dS, T, E, a.db_gate);
  }
  return hipGetLastError();
#undef MOE_TRY
}

}  // namespace moe
