// common.h - types and small device helpers shared by the HIP kernels of the
// MoE layer forward (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kMaxExperts = 256;   // routed experts per layer
constexpr int kWave = 64;          // CDNA wavefront width

// bfloat16 storage is the upper 16 bits of an IEEE float32.
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// float32 -> bfloat16, round to nearest, ties to even; NaN stays NaN: the
// gfx950 conversion instruction (v_cvt_pk_bf16_f32), two values per
// instruction.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return static_cast<uint16_t>(pack_bf16x2(f, 0.0f));
}

// GELU x * Phi(x) = x (1 + erf(x / sqrt 2)) / 2 in fp32, erf from
// Abramowitz & Stegun, Handbook of Mathematical Functions (1964), formula
// 7.1.26: for z >= 0, 1 - erf(z) = (a1 t + a2 t^2 + a3 t^3 + a4 t^4 +
// a5 t^5) exp(-z^2), t = 1 / (1 + p z), with |error| <= 1.5e-7.  With q that
// product at z = |x| / sqrt 2: x < 0 gives x q / 2 (the erfc form, no
// cancellation), x >= 0 gives x - x q / 2.  Measured in fp32 against the
// fp64 definition: |error| <= 3.3e-7 |x| over [-12, 12] (an fp32 erf used
// as 1 + erf loses up to 4.5e-7 in the negative tail), far below the bf16
// rounding of the hidden activations; about a third of the instructions of
// the library erff.
__device__ __forceinline__ float gelu_f32(float a) {
  const float z = fabsf(a) * 0.70710678118654752440f;
  const float t = __builtin_amdgcn_rcpf(__builtin_fmaf(0.3275911f, z, 1.0f));
  float poly = __builtin_fmaf(1.061405429f, t, -1.453152027f);
  poly = __builtin_fmaf(poly, t, 1.421413741f);
  poly = __builtin_fmaf(poly, t, -0.284496736f);
  poly = __builtin_fmaf(poly, t, 0.254829592f);
  const float q = poly * t * __expf(-z * z);
  const float h = 0.5f * a * q;
  return a < 0.0f ? h : a - h;
}

// SiLU x * sigmoid(x) in fp32, the reciprocal from v_rcp_f32 (1 ulp) rather
// than an IEEE division (about twice the instructions).
__device__ __forceinline__ float silu_f32(float g) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
}

__device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

// s_waitcnt immediates (gfx9 family encoding): vmcnt n (6 bits: [3:0] and
// [15:14]), expcnt not waited for (7), lgkmcnt 0 or not waited for (15).
constexpr int waitcnt_vm_lgkm0(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4); }
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// Inclusive prefix sum across the 64 lanes of a wavefront.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  const int lane = threadIdx.x % kWave;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int n = __shfl_up(v, off);
    if (lane >= off) v += n;
  }
  return v;
}

// Exclusive prefix sum over a workgroup of NT threads (NT/64 <= 64 waves);
// `tmp` is LDS scratch of NT/64 ints.  Returns the exclusive prefix of the
// calling thread and the block total through *total.
template <int NT>
__device__ __forceinline__ int block_exclusive_scan(int v, int *tmp, int *total) {
  constexpr int NW = NT / kWave;
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int inc = wave_inclusive_scan(v);
  if (lane == kWave - 1) tmp[wave] = inc;
  __syncthreads();
  int before = 0, all = 0;
  for (int w = 0; w < NW; ++w) {
    const int t = tmp[w];
    if (w < wave) before += t;
    all += t;
  }
  __syncthreads();
  *total = all;
  return before + inc - v;
}

// Number of expert groups that take part in the expert GEMMs: E routed
// groups, plus the shared always-on expert as group E when present.
struct GroupTable {
  const int32_t *offsets;  // [E + 1] group starts in the grouped rows
  int32_t E;
  int32_t S;
  int32_t T;               // tokens (rows of the shared group)
  int32_t routed_rows;     // T * k

  __device__ __forceinline__ int num_groups() const { return E + S; }
  __device__ __forceinline__ int rows(int g) const {
    return g < E ? offsets[g + 1] - offsets[g] : T;
  }
  // first grouped row (of hidden / y_perm) of group g
  __device__ __forceinline__ int row0(int g) const {
    return g < E ? offsets[g] : routed_rows;
  }
};

}  // namespace moe
