// combine.hip - collect: y[t] = sum_j w[t,j] * y_perm[pos[t*k+j]] (+ shared).
//
// Go book chapter "MoE (Mixture of Experts)", section 2 (Forward): the
// output row accumulates weight * expert output for each kept expert in
// slot order.  A gather (every token reads its k grouped rows) instead of a
// scatter-add keeps the sum deterministic without floating-point atomics.
// The shared always-on expert's row sits at grouped row T*k + t and enters
// with weight 1; a slot dropped by the expert capacity (pos = -1) adds
// nothing.  fp32 accumulation, one rounding to the output dtype.
#include "common.h"

#pragma clang fp contract(off)

namespace moe {

constexpr int kCombineThreads = 256;

template <bool BF16>
__device__ __forceinline__ void widen(const uint4 &v, float (&f)[BF16 ? 8 : 4]) {
  if constexpr (BF16) {
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      f[2 * q] = __uint_as_float(u[q] << 16);
      f[2 * q + 1] = __uint_as_float(u[q] & 0xffff0000u);
    }
  } else {
    f[0] = __uint_as_float(v.x);
    f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z);
    f[3] = __uint_as_float(v.w);
  }
}

// KMAX > 0 (k <= KMAX): every row of a vector column is loaded before the
// sum starts, so the k (+ shared) loads are in flight together instead of one
// after another; KMAX = 0: any k, one row at a time.  Either way the sum is
// the same: slot order, one fp32 fused multiply-add per kept slot, then the
// shared row, one rounding at the end.
template <bool BF16, int KMAX>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(
    const void *__restrict__ y_perm, const int32_t *__restrict__ pos,
    const float *__restrict__ w, int T, int k, int d, int rows, int shared,
    void *__restrict__ y) {
  constexpr int VEC = BF16 ? 8 : 4;   // elements per 16-byte vector
  __shared__ int ps[kMaxExperts];
  __shared__ float wsh[kMaxExperts];
  const int nvec = d / VEC;
  const int routed = T * k;
  const uint4 *yp = reinterpret_cast<const uint4 *>(y_perm);
  for (int t = blockIdx.x; t < T; t += gridDim.x) {
    __syncthreads();
    for (int j = threadIdx.x; j < k; j += kCombineThreads) {
      const int pj = pos[(int64_t)t * k + j];
      ps[j] = pj < 0 ? -1 : min(pj, rows - 1);   // -1: dropped (expert capacity)
      wsh[j] = w[(int64_t)t * k + j];
    }
    __syncthreads();
    for (int i = threadIdx.x; i < nvec; i += kCombineThreads) {
      float acc[VEC];
#pragma unroll
      for (int q = 0; q < VEC; ++q) acc[q] = 0.0f;
      if constexpr (KMAX > 0) {
        uint4 v[KMAX + 1];
#pragma unroll
        for (int j = 0; j < KMAX; ++j) {
          v[j] = make_uint4(0u, 0u, 0u, 0u);
          if (j < k && ps[j] >= 0) v[j] = yp[(int64_t)ps[j] * nvec + i];
        }
        v[KMAX] = make_uint4(0u, 0u, 0u, 0u);
        if (shared) v[KMAX] = yp[(int64_t)(routed + t) * nvec + i];
#pragma unroll
        for (int j = 0; j < KMAX; ++j) {
          if (j < k && ps[j] >= 0) {
            float f[VEC];
            widen<BF16>(v[j], f);
            const float wj = wsh[j];
#pragma unroll
            for (int q = 0; q < VEC; ++q) acc[q] = __builtin_fmaf(wj, f[q], acc[q]);
          }
        }
        if (shared) {
          float f[VEC];
          widen<BF16>(v[KMAX], f);
#pragma unroll
          for (int q = 0; q < VEC; ++q) acc[q] = acc[q] + f[q];
        }
      } else {
        for (int j = 0; j <= k; ++j) {
          int row;
          float wj;
          if (j < k) {
            row = ps[j];
            if (row < 0) continue;
            wj = wsh[j];
          } else {
            if (!shared) break;
            row = routed + t;
            wj = 1.0f;
          }
          float f[VEC];
          widen<BF16>(yp[(int64_t)row * nvec + i], f);
          if (j < k) {
#pragma unroll
            for (int q = 0; q < VEC; ++q) acc[q] = __builtin_fmaf(wj, f[q], acc[q]);
          } else {
#pragma unroll
            for (int q = 0; q < VEC; ++q) acc[q] = acc[q] + f[q];
          }
        }
      }
      uint4 o;
      if constexpr (BF16) {
        o.x = pack_bf16x2(acc[0], acc[1]);
        o.y = pack_bf16x2(acc[2], acc[3]);
        o.z = pack_bf16x2(acc[4], acc[5]);
        o.w = pack_bf16x2(acc[6], acc[7]);
      } else {
        o.x = __float_as_uint(acc[0]);
        o.y = __float_as_uint(acc[1]);
        o.z = __float_as_uint(acc[2]);
        o.w = __float_as_uint(acc[3]);
      }
      reinterpret_cast<uint4 *>(y)[(int64_t)t * nvec + i] = o;
    }
  }
}

hipError_t launch_combine(bool bf16, const void *y_perm, const int32_t *pos,
                          const float *w, int T, int k, int d, int S, void *y,
                          hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int rows = T * k + S * T;
  const int blocks = T < 16384 ? T : 16384;
#define MOE_COMBINE(B, KM) \
  combine_kernel<B, KM><<<blocks, kCombineThreads, 0, s>>>(y_perm, pos, w, T, k, d, rows, S, y)
  if (bf16) {
    if (k <= 2) MOE_COMBINE(true, 2);
    else if (k <= 4) MOE_COMBINE(true, 4);
    else if (k <= 8) MOE_COMBINE(true, 8);
    else MOE_COMBINE(true, 0);
  } else {
    if (k <= 2) MOE_COMBINE(false, 2);
    else if (k <= 8) MOE_COMBINE(false, 8);
    else MOE_COMBINE(false, 0);
  }
#undef MOE_COMBINE
  return hipGetLastError();
}

}  // namespace moe
