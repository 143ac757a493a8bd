// gemm_f32.hip - grouped expert GEMMs for fp32 layers (SIMT FMA).
//
// Same grouped problem as the bf16 MFMA kernels (conditional computation over
// the expert groups of the grouped rows), for layers stored in fp32: a plain
// LDS-tiled SIMT GEMM, 64 x 64 output tile, 4 x 4 outputs per thread, fused
// GELU/SwiGLU/bias epilogue.  The grid is (m-tile bound, n-tiles); the
// workgroup finds its expert group by walking the group sizes.
#include "common.h"

namespace moe {

enum F32Mode { kF32UpGelu = 0, kF32UpSwiglu = 1, kF32Down = 2 };

struct F32Args {
  const int32_t *offsets;
  int E, S, T, routed_rows;
  const float *a_routed, *a_shared;
  int K;
  const float *w, *w_shared;
  int w_rows;
  const float *bias;
  float *c;
  int n_out;
  const int32_t *gather;   // or NULL: routed row p is row gather[p] of a_shared (x)
};

template <int MODE>
__global__ __launch_bounds__(256) void gemm_f32_kernel(F32Args a) {
  constexpr int BM = 64, BN = 64, BK = 16;
  constexpr bool SWI = MODE == kF32UpSwiglu;
  constexpr int NB = SWI ? 2 : 1;
  __shared__ float As[BK][BM + 4];
  __shared__ float Bs[NB][BK][BN + 4];

  // find the group of this m-tile
  const int G = a.E + a.S;
  int mt = blockIdx.x, g = 0, rows = 0, r0 = 0;
  for (; g < G; ++g) {
    if (g < a.E) {
      r0 = min(max(a.offsets[g], 0), a.routed_rows);
      const int r1 = min(max(a.offsets[g + 1], r0), a.routed_rows);
      rows = r1 - r0;
    } else {
      r0 = a.routed_rows;
      rows = a.T;
    }
    const int tg = (rows + BM - 1) / BM;
    if (mt < tg) break;
    mt -= tg;
  }
  if (g >= G) return;
  const int m0 = mt * BM;
  const int n0 = blockIdx.y * BN;
  const float *A = g < a.E ? a.a_routed + (int64_t)r0 * a.K : a.a_shared;
  const float *W = g < a.E ? a.w + (int64_t)g * a.w_rows * a.K : a.w_shared;

  const int tid = threadIdx.x;
  const int tx = tid % 16, ty = tid / 16;
  float acc[NB][4][4] = {};

  for (int k0 = 0; k0 < a.K; k0 += BK) {
    // A tile: 64 rows x 16 -> As[k][m]
    for (int q = tid; q < BM * BK / 4; q += 256) {
      const int r = q / (BK / 4), c = (q % (BK / 4)) * 4;
      const int row = min(m0 + r, rows - 1);
      const float *arow = A + (int64_t)row * a.K;
      if (a.gather && g < a.E) {   // the token's row of x (an index out of range reads row 0)
        const int src = a.gather[r0 + row];
        arow = a.a_shared + (int64_t)((unsigned)src < (unsigned)a.T ? src : 0) * a.K;
      }
      const float4 v = *reinterpret_cast<const float4 *>(arow + k0 + c);
      As[c + 0][r] = v.x; As[c + 1][r] = v.y; As[c + 2][r] = v.z; As[c + 3][r] = v.w;
    }
    for (int b = 0; b < NB; ++b)
      for (int q = tid; q < BN * BK / 4; q += 256) {
        const int r = q / (BK / 4), c = (q % (BK / 4)) * 4;
        const int n = min(n0 + r, a.n_out - 1) + b * a.n_out;   // up half at h + n
        const int wr = SWI ? n : min(n0 + r, a.w_rows - 1);
        const float4 v = *reinterpret_cast<const float4 *>(W + (int64_t)wr * a.K + k0 + c);
        Bs[b][c + 0][r] = v.x; Bs[b][c + 1][r] = v.y; Bs[b][c + 2][r] = v.z; Bs[b][c + 3][r] = v.w;
      }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BK; ++kk) {
      float av[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float bv = Bs[b][kk][tx + 16 * j];
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[b][i][j] = __builtin_fmaf(av[i], bv, acc[b][i][j]);
        }
    }
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty * 4 + i;
    if (m >= rows) continue;
    float *crow = a.c + (int64_t)((g < a.E ? r0 : a.routed_rows) + m) * a.n_out;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx + 16 * j;
      if (n >= a.n_out) continue;
      float v;
      if constexpr (MODE == kF32UpSwiglu) {
        v = silu_f32(acc[0][i][j]) * acc[1][i][j];
      } else {
        const float b = (a.bias && g < a.E) ? a.bias[(int64_t)g * a.n_out + n] : 0.0f;
        v = MODE == kF32UpGelu ? gelu_f32(acc[0][i][j] + b) : acc[0][i][j] + b;
      }
      crow[n] = v;
    }
  }
}

template <int MODE>
static hipError_t launch_f32(const F32Args &a, hipStream_t s) {
  const int mt_bound = (a.routed_rows + 63) / 64 + a.E + a.S;
  dim3 grid(mt_bound, (a.n_out + 63) / 64);
  gemm_f32_kernel<MODE><<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_expert_up_f32(bool swiglu, const int32_t *offsets, int E, int S,
                                int T, int k, int d, int h, const void *x_perm,
                                const int32_t *perm_src, const void *x, const void *w_up,
                                const void *w_up_shared, const void *b_up,
                                void *hidden, hipStream_t s) {
  F32Args a{};
  if (!x_perm) a.gather = perm_src;   // token rows gathered from x
  a.offsets = offsets; a.E = E; a.S = S; a.T = T; a.routed_rows = T * k;
  a.a_routed = static_cast<const float *>(x_perm ? x_perm : x);
  a.a_shared = static_cast<const float *>(x);
  a.K = d;
  a.w = static_cast<const float *>(w_up);
  a.w_shared = static_cast<const float *>(w_up_shared);
  a.w_rows = swiglu ? 2 * h : h;
  a.bias = static_cast<const float *>(b_up);
  a.c = static_cast<float *>(hidden);
  a.n_out = h;
  return swiglu ? launch_f32<kF32UpSwiglu>(a, s) : launch_f32<kF32UpGelu>(a, s);
}

hipError_t launch_expert_down_f32(const int32_t *offsets, int E, int S, int T,
                                  int k, int d, int h, const void *hidden,
                                  const void *w_down, const void *w_down_shared,
                                  const void *b_down, void *y_perm,
                                  hipStream_t s) {
  F32Args a{};
  a.offsets = offsets; a.E = E; a.S = S; a.T = T; a.routed_rows = T * k;
  a.a_routed = static_cast<const float *>(hidden);
  a.a_shared = static_cast<const float *>(hidden) + (int64_t)T * k * h;
  a.K = h;
  a.w = static_cast<const float *>(w_down);
  a.w_shared = static_cast<const float *>(w_down_shared);
  a.w_rows = d;
  a.bias = static_cast<const float *>(b_down);
  a.c = static_cast<float *>(y_perm);
  a.n_out = d;
  return launch_f32<kF32Down>(a, s);
}

}  // namespace moe
