// noisy.hip - noisy top-k gating (the training-time gate) and the smooth
// load estimate.
//
// "Sparsely-Gated MoE" Qiita summary, "Gating: Noisy Top-k Softmax": during
// training the score of expert i is H_i = (x W_g)_i + n_i Softplus((x
// W_noise)_i) with n_i ~ N(0, 1), and G = softmax(KeepTopK(H, k)).  The
// clean and the noise scores are the router's own fp32 chains (route.hip,
// run once with W_g and its bias, once with W_noise and no bias); this file
// takes it from there, one wavefront per token:
//   Softplus in double from the fp32 noise score, rounded to fp32;
//   H = fma(n, Softplus, clean) in fp32 (one rounding), so the selection is
//   taken in fp32 like the clean gate's;
//   stable top-k of H (ties to the lower index), softmax over the kept H;
//   the smooth load term (same summary, "Load-balancing losses", which
//   calls Load(X) a smooth estimate of the per-expert sample count; the
//   estimator is Shazeer et al.'s): P(x, i) = Phi((clean_i - t_i) /
//   Softplus_i), t_i the k-th largest H without entry i, which is the
//   (k+1)-th largest H when i is kept and the k-th largest otherwise.
// Importance and Load are summed per workgroup in a fixed order, then over
// workgroups in a fixed order by one wavefront per expert: deterministic.
#include "common.h"

#pragma clang fp contract(off)

namespace moe {

constexpr int kNoisyThreads = 256;
constexpr int kNoisyWaves = kNoisyThreads / kWave;
constexpr int kNoisyTPB = 16;   // tokens per workgroup, 4 per wavefront

__device__ __forceinline__ double softplus_d(double v) {
  return v > 0.0 ? v + log1p(exp(-v)) : log1p(exp(v));
}

// part: [gridDim.x][2][E] fp32 (Importance, Load) per workgroup.
template <int NQ>
__global__ __launch_bounds__(kNoisyThreads) void noisy_topk_kernel(
    const float *__restrict__ noise, int T, int E, int k,
    const float *__restrict__ clean, float *__restrict__ scale,
    int32_t *__restrict__ topk_idx, float *__restrict__ topk_w,
    int32_t *__restrict__ counts, float *__restrict__ part) {
  __shared__ float simp[kNoisyWaves][kMaxExperts];
  __shared__ float sload[kNoisyWaves][kMaxExperts];
  __shared__ int cnt[kMaxExperts];
  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = tid / kWave;
  for (int i = tid; i < kMaxExperts; i += kNoisyThreads) {
    cnt[i] = 0;
#pragma unroll
    for (int w = 0; w < kNoisyWaves; ++w) {
      simp[w][i] = 0.0f;
      sload[w][i] = 0.0f;
    }
  }
  __syncthreads();

  for (int r = wave; r < kNoisyTPB; r += kNoisyWaves) {
    const int t = blockIdx.x * kNoisyTPB + r;
    if (t >= T) break;
    const int64_t row = (int64_t)t * E;
    float c[NQ], s[NQ], h[NQ];
    uint32_t avail = 0;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int e = lane + 64 * q;
      c[q] = s[q] = h[q] = 0.0f;
      if (e < E) {
        c[q] = clean[row + e];
        s[q] = (float)softplus_d((double)scale[row + e]);
        scale[row + e] = s[q];
        h[q] = __builtin_fmaf(noise[row + e], s[q], c[q]);
        avail |= 1u << q;
      }
    }
    // k (+1 when k < E) rounds of a 64-lane arg-max under (H desc, index asc)
    int my_e[NQ];
    float my_v[NQ];
    uint32_t kept = 0;
    float s0 = 0.0f, vk = 0.0f, vk1 = 0.0f;
    const int rounds = k < E ? k + 1 : k;
    for (int j = 0; j < rounds; ++j) {
      float bv = 0.0f;
      int be = 0x7fffffff;
#pragma unroll
      for (int q = 0; q < NQ; ++q)
        if ((avail >> q) & 1u)
          if (be == 0x7fffffff || h[q] > bv) {
            bv = h[q];
            be = lane + 64 * q;
          }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        const float ov = __shfl_xor(bv, off);
        const int oe = __shfl_xor(be, off);
        const bool take = oe != 0x7fffffff &&
                          (be == 0x7fffffff || ov > bv || (ov == bv && oe < be));
        if (take) {
          bv = ov;
          be = oe;
        }
      }
      if (j == k) {
        vk1 = bv;
        break;
      }
      if ((be & 63) == lane) {
        avail &= ~(1u << (be >> 6));
        kept |= 1u << (be >> 6);
      }
      if (j == 0) s0 = bv;
      if (j == k - 1) vk = bv;
#pragma unroll
      for (int q = 0; q < NQ; ++q)
        if (j == lane + 64 * q) {
          my_e[q] = be;
          my_v[q] = bv;
        }
    }
    // softmax over the kept H
    float z[NQ];
    float sum = 0.0f;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      z[q] = 0.0f;
      if (lane + 64 * q < k) {
        z[q] = expf(my_v[q] - s0);
        sum += z[q];
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int j = lane + 64 * q;
      if (j < k) {
        const float wj = z[q] / sum;
        topk_idx[(int64_t)t * k + j] = my_e[q];
        topk_w[(int64_t)t * k + j] = wj;
        simp[wave][my_e[q]] += wj;   // the kept experts of a token are distinct
        atomicAdd(&cnt[my_e[q]], 1);
      }
    }
    // smooth load terms of this token's experts
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int e = lane + 64 * q;
      if (e < E) {
        double p = 1.0;
        if (k < E) {
          const double thr = (double)(((kept >> q) & 1u) ? vk1 : vk);
          const double diff = (double)c[q] - thr;
          p = s[q] == 0.0f ? (diff > 0.0 ? 1.0 : 0.0)
                           : 0.5 * erfc(-(diff / (double)s[q]) * M_SQRT1_2);
        }
        sload[wave][e] += (float)p;
      }
    }
  }
  __syncthreads();
  float *out = part + (int64_t)blockIdx.x * 2 * E;
  for (int e = tid; e < E; e += kNoisyThreads) {
    float a = 0.0f, b = 0.0f;
#pragma unroll
    for (int w = 0; w < kNoisyWaves; ++w) {
      a += simp[w][e];
      b += sload[w][e];
    }
    out[e] = a;
    out[E + e] = b;
    if (cnt[e]) atomicAdd(counts + e, cnt[e]);
  }
}

// One wavefront per expert: lane l sums the partials of workgroups l, l+64,
// ... in order (fp64), then a fixed butterfly; sums[e] and sums[E+e] keep
// the fp64 totals for the CV^2 kernel.
__global__ __launch_bounds__(kWave) void noisy_reduce_kernel(
    const float *__restrict__ part, int nblk, int E, float *__restrict__ importance,
    float *__restrict__ load, double *__restrict__ sums) {
  const int e = blockIdx.x;
  const int lane = threadIdx.x;
  double a = 0.0, b = 0.0;
  for (int blk = lane; blk < nblk; blk += kWave) {
    a += part[(int64_t)blk * 2 * E + e];
    b += part[(int64_t)blk * 2 * E + E + e];
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    a += __shfl_xor(a, off);
    b += __shfl_xor(b, off);
  }
  if (lane == 0) {
    importance[e] = (float)a;
    load[e] = (float)b;
    sums[e] = a;
    sums[E + e] = b;
  }
}

// CV^2 of Importance and of Load (population variance / mean^2, 0 when the
// mean is 0) from the fp64 totals, in expert order.
__global__ void noisy_cv2_kernel(const double *__restrict__ sums, int E, double *__restrict__ cv2) {
  if (threadIdx.x != 0) return;
  double ma = 0.0, mb = 0.0;
  for (int i = 0; i < E; ++i) {
    ma += sums[i];
    mb += sums[E + i];
  }
  ma /= E;
  mb /= E;
  double va = 0.0, vb = 0.0;
  for (int i = 0; i < E; ++i) {
    va += (sums[i] - ma) * (sums[i] - ma);
    vb += (sums[E + i] - mb) * (sums[E + i] - mb);
  }
  va /= E;
  vb /= E;
  cv2[0] = ma == 0.0 ? 0.0 : va / (ma * ma);
  cv2[1] = mb == 0.0 ? 0.0 : vb / (mb * mb);
}

__global__ void noisy_zero_kernel(float *importance, float *load, int E, double *cv2) {
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    importance[e] = 0.0f;
    load[e] = 0.0f;
  }
  if (threadIdx.x == 0 && cv2) {
    cv2[0] = 0.0;
    cv2[1] = 0.0;
  }
}

// Workspace: the fp64 totals [2E], then the partials [nblk][2][E] fp32.
int64_t noisy_workspace_bytes(int64_t T, int E) {
  const int64_t nblk = (T + kNoisyTPB - 1) / kNoisyTPB;
  return 2 * E * (int64_t)sizeof(double) + nblk * 2 * E * (int64_t)sizeof(float);
}

hipError_t launch_fill_i32(int32_t *p, int n, int32_t v, hipStream_t s);

// After the clean scores (clean) and the raw noise scores (in scale) are
// written: zero the counts, then the gate and the reduction.
hipError_t launch_noisy_gate(const float *noise, int T, int E, int k, const float *clean,
                             float *scale, int32_t *idx, float *w, int32_t *counts,
                             float *importance, float *load, double *cv2, void *ws,
                             hipStream_t s) {
  hipError_t err = launch_fill_i32(counts, E, 0, s);
  if (err != hipSuccess) return err;
  if (T == 0) {
    noisy_zero_kernel<<<1, kMaxExperts, 0, s>>>(importance, load, E, cv2);
    return hipGetLastError();
  }
  const int nblk = (T + kNoisyTPB - 1) / kNoisyTPB;
  double *sums = static_cast<double *>(ws);
  float *part = reinterpret_cast<float *>(sums + 2 * E);
  if (E <= 64)
    noisy_topk_kernel<1><<<nblk, kNoisyThreads, 0, s>>>(noise, T, E, k, clean, scale, idx, w,
                                                        counts, part);
  else if (E <= 128)
    noisy_topk_kernel<2><<<nblk, kNoisyThreads, 0, s>>>(noise, T, E, k, clean, scale, idx, w,
                                                        counts, part);
  else
    noisy_topk_kernel<4><<<nblk, kNoisyThreads, 0, s>>>(noise, T, E, k, clean, scale, idx, w,
                                                        counts, part);
  noisy_reduce_kernel<<<E, kWave, 0, s>>>(part, nblk, E, importance, load, sums);
  if (cv2) noisy_cv2_kernel<<<1, kWave, 0, s>>>(sums, E, cv2);
  return hipGetLastError();
}

}  // namespace moe
