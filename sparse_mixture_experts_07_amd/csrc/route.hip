// route.hip - router scores, KeepTopK and the softmax over the kept scores.
//
// One workgroup owns BT = 32 tokens and every expert.  The score of (t, e) is
// one fp32 fused multiply-add chain over i = 0..d-1 in ascending order,
// starting from +0, with the router bias added after the last term: the Go
// book chapter "MoE (Mixture of Experts)", section 2 (Route) accumulates
// score += x_i * W_g[i, e] one term at a time in float32.  Tokens and
// experts are spread over the threads; every thread keeps its chains in
// registers, so no chain is ever split or reordered.
//
// Selection: the first k entries of a stable descending sort, i.e. the k
// largest scores with equal scores ordered by the lower expert index (same
// section, sort.SliceStable; KeepTopK of the "Sparsely-Gated MoE" Qiita
// summary, "Gating: Noisy Top-k Softmax").  One wavefront per token runs k
// rounds of a 64-lane arg-max whose order is (score desc, index asc).
// Weights: exp(s_j - s_0) / sum_i exp(s_i - s_0) over the kept scores only
// (default gate mode).  Two more gate modes take the same selection: the
// bias steers the selection only and the weights are the softmax of the
// unbiased kept scores (the Go chapter on DeepSeek-V3's bias balancing,
// section 3 and "Pros, cons and real examples"), or the softmax runs over
// all E scores and is read at the kept experts without renormalisation
// (techfeed summary, "The hardest part: making the router trainable").
// Counts: an LDS histogram per workgroup, then one integer atomic per
// (workgroup, expert), so counts are exact and order-independent.
#include "common.h"

#pragma clang fp contract(off)

namespace moe {

constexpr int kRouteThreads = 256;
constexpr int kRouteBK = 32;
constexpr int kGateTopK = 0;         // softmax over the kept scores
constexpr int kGateBiasSelects = 1;  // softmax over the kept unbiased scores
constexpr int kGateSoftmaxAll = 2;   // softmax over all scores, not renormalised

// Gate value of lane e's kept slot inside one EP-lane group that holds one
// token: lane e carries expert e's biased score sc and unbiased chain acc;
// after KeepTopK, lanes j < k carry the j-th kept expert my_e and its
// biased score my_v, and s0 is the largest score.  Every lane of the group
// takes part in the shuffles; lanes j >= k return an unused value.
template <int EP>
__device__ __forceinline__ float group_gate(int gate, int e, int E, int k, float sc,
                                            float acc, int my_e, float my_v, float s0) {
  if (gate == kGateSoftmaxAll) {
    float all = e < E ? expf(sc - s0) : 0.0f;
#pragma unroll
    for (int off = EP / 2; off >= 1; off >>= 1) all += __shfl_xor(all, off);
    return (e < k ? expf(my_v - s0) : 0.0f) / all;
  }
  float z;
  if (gate == kGateBiasSelects) {
    const float r = __shfl(acc, my_e, EP);   // unbiased score of the kept expert
    float m = e < k ? r : -INFINITY;
#pragma unroll
    for (int off = EP / 2; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    z = e < k ? expf(r - m) : 0.0f;
  } else {
    z = e < k ? expf(my_v - s0) : 0.0f;
  }
  float sum = z;
#pragma unroll
  for (int off = EP / 2; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
  return z / sum;
}

template <typename XT>
struct XLoad;

template <>
struct XLoad<uint16_t> {  // bf16 rows: 8 values (16 B) per load
  static constexpr int kVec = 8;
  __device__ static void load(const uint16_t *p, float *out) {
    uint4 v = *reinterpret_cast<const uint4 *>(p);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = __uint_as_float(w[i] << 16);
      out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
};

template <>
struct XLoad<float> {  // fp32 rows: 4 values (16 B) per load
  static constexpr int kVec = 4;
  __device__ static void load(const float *p, float *out) {
    float4 v = *reinterpret_cast<const float4 *>(p);
    out[0] = v.x; out[1] = v.y; out[2] = v.z; out[3] = v.w;
  }
};

// TX threads across experts (each owns EPT experts strided by TX), TY =
// 256/TX threads across tokens (each owns TPT consecutive tokens).  The K
// loop stages "super-chunks" of G x 32 columns of x and W_g in LDS (k
// contiguous, rows padded by 16 B against bank conflicts), double-buffered:
// the global loads of super-chunk c+1 fly while super-chunk c is consumed,
// so one load latency is paid per G x 32 columns.  Each thread walks k in
// ascending order for every one of its TPT x EPT chains.
template <typename XT, int TX, int EPT, int TPT, int GMAX, int NTH>
__global__ __launch_bounds__(NTH) void route_kernel(
    const XT *__restrict__ x, const float *__restrict__ wg,
    const float *__restrict__ bg, int T, int d, int E, int k, int gate, int G,
    int32_t *__restrict__ topk_idx, float *__restrict__ topk_w,
    int32_t *__restrict__ counts, float *__restrict__ logits) {
  constexpr int TY = NTH / TX;
  constexpr int BT = TY * TPT;
  constexpr int EP = TX * EPT;      // padded expert count
  constexpr int EPS = EP + 1;       // score row stride
  constexpr int BK = kRouteBK;
  constexpr int KS = BK + 4;        // staged row stride (floats)
  constexpr int NQ = (EP + 63) / 64;  // score slots per lane in the top-k
  constexpr int VEC = XLoad<XT>::kVec;
  constexpr int XQ = BT * (BK / VEC);              // x vector loads per chunk
  constexpr int XL = (XQ + NTH - 1) / NTH;
  constexpr int WQ = EP * (BK / 4);                // W_g float4 loads per chunk
  constexpr int WL = (WQ + NTH - 1) / NTH;
  constexpr int CHUNK = (BT + EP) * KS;            // floats per staged chunk

  extern __shared__ float lds[];                   // 2 * G * CHUNK floats
  __shared__ int cnt[EP];
  const int stage = G * CHUNK;

  const int tid = threadIdx.x;
  const int tx = tid % TX;
  const int ty = tid / TX;
  const int t0 = blockIdx.x * BT;

  for (int e = tid; e < EP; e += NTH) cnt[e] = 0;

  float acc[TPT][EPT];
#pragma unroll
  for (int r = 0; r < TPT; ++r)
#pragma unroll
    for (int j = 0; j < EPT; ++j) acc[r][j] = 0.0f;

  float xr[GMAX][XL][VEC];
  float4 wr[GMAX][WL];
  auto gload = [&](int k0) {   // super-chunk starting at column k0
#pragma unroll
    for (int g = 0; g < GMAX; ++g) {
      if (g >= G) break;
      const int kg = k0 + g * BK;
#pragma unroll
      for (int i = 0; i < XL; ++i) {
        const int q = tid + i * NTH;
        const int row = q / (BK / VEC);
        const int c = (q % (BK / VEC)) * VEC;
        if (q < XQ && t0 + row < T) {
          XLoad<XT>::load(x + (int64_t)(t0 + row) * d + kg + c, xr[g][i]);
        } else {
#pragma unroll
          for (int v = 0; v < VEC; ++v) xr[g][i][v] = 0.0f;
        }
      }
#pragma unroll
      for (int i = 0; i < WL; ++i) {
        const int q = tid + i * NTH;
        const int e = q / (BK / 4);
        const int c = (q % (BK / 4)) * 4;
        wr[g][i] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (q < WQ && e < E) wr[g][i] = *reinterpret_cast<const float4 *>(wg + (int64_t)e * d + kg + c);
      }
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int g = 0; g < GMAX; ++g) {
      if (g >= G) break;
      float *xs = lds + buf * stage + g * CHUNK;
      float *ws = xs + BT * KS;
#pragma unroll
      for (int i = 0; i < XL; ++i) {
        const int q = tid + i * NTH;
        if (q < XQ) {
          const int row = q / (BK / VEC);
          const int c = (q % (BK / VEC)) * VEC;
#pragma unroll
          for (int v = 0; v < VEC; v += 4)
            *reinterpret_cast<float4 *>(xs + row * KS + c + v) =
                make_float4(xr[g][i][v], xr[g][i][v + 1], xr[g][i][v + 2], xr[g][i][v + 3]);
        }
      }
#pragma unroll
      for (int i = 0; i < WL; ++i) {
        const int q = tid + i * NTH;
        if (q < WQ) *reinterpret_cast<float4 *>(ws + (q / (BK / 4)) * KS + (q % (BK / 4)) * 4) = wr[g][i];
      }
    }
  };
  auto consume = [&](int buf) {
    for (int g = 0; g < G; ++g) {
      const float *xs = lds + buf * stage + g * CHUNK;
      const float *ws = xs + BT * KS;
#pragma unroll
      for (int kk = 0; kk < BK; kk += 4) {
        float4 xv[TPT], wv[EPT];
#pragma unroll
        for (int r = 0; r < TPT; ++r)
          xv[r] = *reinterpret_cast<const float4 *>(xs + (ty * TPT + r) * KS + kk);
#pragma unroll
        for (int j = 0; j < EPT; ++j)
          wv[j] = *reinterpret_cast<const float4 *>(ws + (tx + TX * j) * KS + kk);
#pragma unroll
        for (int r = 0; r < TPT; ++r)
#pragma unroll
          for (int j = 0; j < EPT; ++j) {
            float a = acc[r][j];
            a = __builtin_fmaf(xv[r].x, wv[j].x, a);
            a = __builtin_fmaf(xv[r].y, wv[j].y, a);
            a = __builtin_fmaf(xv[r].z, wv[j].z, a);
            a = __builtin_fmaf(xv[r].w, wv[j].w, a);
            acc[r][j] = a;
          }
      }
    }
  };

  const int nsc = d / (BK * G);
  gload(0);
  lstore(0);
  __syncthreads();
  for (int sc = 0; sc < nsc; ++sc) {
    const int buf = sc & 1;
    const bool more = sc + 1 < nsc;
    if (more) gload((sc + 1) * BK * G);
    // keep the loads ahead of the arithmetic (not sunk next to their stores)
    __builtin_amdgcn_sched_barrier(0);
    consume(buf);
    __builtin_amdgcn_sched_barrier(0);
    if (more) lstore(buf ^ 1);
    __syncthreads();
  }
  float(*ls)[EPS] = reinterpret_cast<float(*)[EPS]>(lds);
  float(*lr)[EPS] = reinterpret_cast<float(*)[EPS]>(lds + BT * EPS);  // unbiased

#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    const int e = tx + TX * j;
    if (e >= E) continue;
    const float b = bg ? bg[e] : 0.0f;
#pragma unroll
    for (int r = 0; r < TPT; ++r) {
      const int row = ty * TPT + r;
      const float s = bg ? acc[r][j] + b : acc[r][j];
      ls[row][e] = s;
      if (gate == kGateBiasSelects) lr[row][e] = acc[r][j];
      if (logits && t0 + row < T) logits[(int64_t)(t0 + row) * E + e] = s;
    }
  }
  __syncthreads();

  // ---- KeepTopK + softmax: one wavefront per token ----
  const int lane = tid % kWave;
  const int wave = tid / kWave;
  constexpr int NW = NTH / kWave;
  for (int row = wave; row < BT; row += NW) {
    const int t = t0 + row;
    if (t >= T) break;
    float v[NQ];
    uint32_t avail = 0;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int e = lane + 64 * q;
      v[q] = 0.0f;
      if (e < E) {
        v[q] = ls[row][e];
        avail |= 1u << q;
      }
    }
    int my_e[NQ];
    float my_v[NQ];
    float s0 = 0.0f;
    for (int j = 0; j < k; ++j) {
      // lane-local best: strictly greater wins, so the lower index (lower q)
      // keeps a tie
      float bv = 0.0f;
      int be = 0x7fffffff;
#pragma unroll
      for (int q = 0; q < NQ; ++q)
        if ((avail >> q) & 1u)
          if (be == 0x7fffffff || v[q] > bv) {
            bv = v[q];
            be = lane + 64 * q;
          }
      // wave arg-max under (score desc, index asc); a total order, so every
      // lane ends with the same winner
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
      if ((be & 63) == lane) avail &= ~(1u << (be >> 6));
      if (j == 0) s0 = bv;
#pragma unroll
      for (int q = 0; q < NQ; ++q)
        if (j == lane + 64 * q) {
          my_e[q] = be;
          my_v[q] = bv;
        }
    }
    float z[NQ];
    float part = 0.0f;
    if (gate == kGateBiasSelects) {
      // softmax of the unbiased scores of the kept experts
      float m = -INFINITY;
#pragma unroll
      for (int q = 0; q < NQ; ++q)
        if (lane + 64 * q < k) {
          my_v[q] = lr[row][my_e[q]];
          m = fmaxf(m, my_v[q]);
        }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
      s0 = m;
    }
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      z[q] = 0.0f;
      if (lane + 64 * q < k) {
        z[q] = expf(my_v[q] - s0);
        if (gate != kGateSoftmaxAll) part += z[q];
      }
    }
    if (gate == kGateSoftmaxAll) {
      // denominator over all E scores
#pragma unroll
      for (int q = 0; q < NQ; ++q)
        if (lane + 64 * q < E) part += expf(ls[row][lane + 64 * q] - s0);
    }
    // butterfly sum: fp32 addition is commutative, so all lanes agree
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) part += __shfl_xor(part, off);
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int j = lane + 64 * q;
      if (j < k) {
        topk_idx[(int64_t)t * k + j] = my_e[q];
        topk_w[(int64_t)t * k + j] = z[q] / part;
        atomicAdd(&cnt[my_e[q]], 1);
      }
    }
  }
  __syncthreads();
  for (int e = tid; e < E; e += NTH)
    if (counts && cnt[e]) atomicAdd(counts + e, cnt[e]);
}

__global__ void fill_i32_kernel(int32_t *p, int n, int32_t v) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x)
    p[i] = v;
}

// The end of every chain layout with one (token, expert) chain per lane:
// lane (t, e) holds the unbiased chain acc of its token and expert, the EP
// lanes of token t form one group.  Biased score, logits, KeepTopK over the
// group (lower index wins ties), gate weights, outputs, and the workgroup's
// count histogram cnt[] (zeroed by the caller before this point; NTH
// threads) merged into counts with one atomic per (workgroup, expert).
template <int EP, int NTH>
__device__ __forceinline__ void lane_select(float acc, int t, int e, int T, int E, int k,
                                            int gate, const float *__restrict__ bg,
                                            int32_t *__restrict__ topk_idx,
                                            float *__restrict__ topk_w,
                                            int32_t *__restrict__ counts,
                                            float *__restrict__ logits, int *cnt) {
  const bool valid = t < T && e < E;
  float sc = acc;
  if (bg && e < E) sc = acc + bg[e];
  if (logits && valid) logits[(int64_t)t * E + e] = sc;

  bool avail = e < E;
  int my_e = 0;
  float my_v = 0.0f, s0 = 0.0f;
  for (int j = 0; j < k; ++j) {
    float bv = sc;
    int be = avail ? e : 0x7fffffff;
#pragma unroll
    for (int off = EP / 2; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off);
      const int oe = __shfl_xor(be, off);
      const bool take = oe != 0x7fffffff &&
                        (be == 0x7fffffff || ov > bv || (ov == bv && oe < be));
      if (take) {
        bv = ov;
        be = oe;
      }
    }
    if (be == e) avail = false;
    if (j == 0) s0 = bv;
    if (e == j) {
      my_e = be;
      my_v = bv;
    }
  }
  const float gw = group_gate<EP>(gate, e, E, k, sc, acc, my_e, my_v, s0);
  __syncthreads();   // cnt[] zeroed
  if (t < T && e < k) {
    topk_idx[(int64_t)t * k + e] = my_e;
    topk_w[(int64_t)t * k + e] = gw;
    atomicAdd(&cnt[my_e], 1);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < E; i += NTH)
    if (counts && cnt[i]) atomicAdd(counts + i, cnt[i]);
}

// ---------------------------------------------------------------------------
// Few experts (E <= 64): a wavefront owns 64/EP tokens x EP experts with one
// (token, expert) chain per lane, and streams its x and W_g rows straight
// from memory through buffer loads (reads past a row's end or past the last
// token return zeros).  Four register sets of 32 columns rotate: a set is
// refilled right after it is consumed, so three sets (96 columns of
// arithmetic) cover each load's latency.  No LDS staging, no barriers in the
// K loop.  KeepTopK/softmax run inside each EP-lane group with shuffles.
template <typename XT>
struct RowLoad;
template <>
struct RowLoad<uint16_t> {   // 32 bf16 columns = 4 x 16 B
  static constexpr int kLoads = 4;
  static constexpr int kBytes = 2;
  __device__ static void expand(const u32x4_t (&v)[kLoads], float *out) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        out[8 * i + 2 * q] = __uint_as_float(v[i][q] << 16);
        out[8 * i + 2 * q + 1] = __uint_as_float(v[i][q] & 0xffff0000u);
      }
  }
};
template <>
struct RowLoad<float> {      // 32 fp32 columns = 8 x 16 B
  static constexpr int kLoads = 8;
  static constexpr int kBytes = 4;
  __device__ static void expand(const u32x4_t (&v)[kLoads], float *out) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) out[4 * i + q] = __uint_as_float(v[i][q]);
  }
};

constexpr int kBufWord3 = 0x00020000;   // raw buffer resource, gfx9 family

template <typename XT, int EP, int NTH>
__global__ __launch_bounds__(NTH) void route_direct_kernel(
    const XT *__restrict__ x, const float *__restrict__ wg,
    const float *__restrict__ bg, int T, int d, int E, int k, int gate,
    int32_t *__restrict__ topk_idx, float *__restrict__ topk_w,
    int32_t *__restrict__ counts, float *__restrict__ logits) {
  constexpr int TPW = kWave / EP;          // tokens per wavefront
  constexpr int NS = 4;                    // rotating register sets
  constexpr int XL = RowLoad<XT>::kLoads;  // x loads per 32 columns
  __shared__ int cnt[EP];
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int e = lane % EP;
  const int t = (blockIdx.x * (NTH / kWave) + wave) * TPW + lane / EP;
  for (int i = threadIdx.x; i < EP; i += NTH) cnt[i] = 0;

  const uint32_t xrec = (uint32_t)T * (uint32_t)d * RowLoad<XT>::kBytes;
  const uint32_t wrec = (uint32_t)E * (uint32_t)d * 4u;
  const __amdgpu_buffer_rsrc_t rx =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<XT *>(x), 0, xrec, kBufWord3);
  const __amdgpu_buffer_rsrc_t rw =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(wg), 0, wrec, kBufWord3);
  // a lane without a chain reads only out-of-range zeros
  const uint32_t xo = t < T ? (uint32_t)t * (uint32_t)d * RowLoad<XT>::kBytes : xrec;
  const uint32_t wo = e < E ? (uint32_t)e * (uint32_t)d * 4u : wrec;

  u32x4_t xs[NS][XL], ws[NS][8];
  auto load = [&](int set, int c0) {   // columns c0 .. c0+31
#pragma unroll
    for (int i = 0; i < XL; ++i)
      xs[set][i] = __builtin_amdgcn_raw_buffer_load_b128(
          rx, xo + (uint32_t)c0 * RowLoad<XT>::kBytes + 16u * i, 0, 0);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      ws[set][i] = __builtin_amdgcn_raw_buffer_load_b128(rw, wo + (uint32_t)c0 * 4u + 16u * i, 0, 0);
  };
  float acc = 0.0f;
  auto consume = [&](int set) {
    float xv[32];
    RowLoad<XT>::expand(xs[set], xv);
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) acc = __builtin_fmaf(xv[4 * i + q], __uint_as_float(ws[set][i][q]), acc);
  };
#pragma unroll
  for (int u = 0; u < NS; ++u) load(u, 32 * u);
  const int nstep = d / 32;   // d is a multiple of 64
  int c = 0;
  for (; c + NS <= nstep; c += NS) {
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      consume(u);
      __builtin_amdgcn_sched_barrier(0);
      load(u, 32 * (c + u + NS));   // past the row end: never consumed
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int u = 0; u < NS; ++u)
    if (c + u < nstep) consume(u);

  lane_select<EP, NTH>(acc, t, e, T, E, k, gate, bg, topk_idx, topk_w, counts, logits, cnt);
}

// Workgroups of four wavefronts; one wavefront each when there are fewer
// wavefronts than CUs (decode batches), so that the chains and their operand
// streams spread over as many CUs as possible.
// ---------------------------------------------------------------------------
// The same chains (one (token, expert) chain per lane, EP-lane groups per
// token), with the operands staged in LDS: each workgroup of NWV wavefronts
// (TPB tokens x EP experts) brings chunks of CC columns of its x rows and of
// W_g into four rotating LDS buffers with buffer loads that write LDS
// directly, three chunks ahead of the chains, so load latency is hidden
// without holding prefetched operands in registers, and every x or W_g
// element crosses the memory pipeline once per workgroup instead of once
// per lane that uses it.  A chain reads its 32-column slices from LDS; the
// 16-byte slots of each row are XOR-swizzled so that the lanes of a
// wavefront, reading the same column of up to 16 rows, hit distinct banks.
template <typename XT, int EP, int NWV>
struct LaneGeom {
  static constexpr int NTH = NWV * kWave;
  static constexpr int TPB = NWV * (kWave / EP);         // tokens per workgroup
  static constexpr int BPC = TPB * (int)sizeof(XT) + EP * 4;   // bytes per column
  static constexpr int CC0 = 24576 / BPC;
  static constexpr int CC = CC0 >= 256 ? 256 : CC0 >= 128 ? 128 : CC0 >= 64 ? 64 : 32;
  static constexpr int XS = CC * (int)sizeof(XT) / 16;   // 16-byte slots of an x row segment
  static constexpr int WS = CC * 4 / 16;                 // ... of a W_g row segment
  static constexpr int XM = XS < 16 ? XS : 16;           // swizzle ranges
  static constexpr int WM = WS < 16 ? WS : 16;
  static constexpr int XBLK = (TPB * XS + 63) / 64;      // 1 KB DMA blocks per chunk
  static constexpr int WBLK = (EP * WS + 63) / 64;
  static constexpr int NBLK = XBLK + WBLK;
  static constexpr int BPW = (NBLK + NWV - 1) / NWV;     // per wavefront (last repeats)
  static constexpr int CHUNK = NBLK * 1024;              // LDS bytes per buffer
  static constexpr int NB = 4;
  static_assert(2 * BPW < 64, "vmcnt range");
  static __device__ __forceinline__ int xslot(int r, int j) { return r * XS + (j ^ (r % XM)); }
  static __device__ __forceinline__ int wslot(int r, int j) { return r * WS + (j ^ (r % WM)); }
};

template <typename XT, int EP, int NWV>
__global__ __launch_bounds__(NWV * kWave) void route_lane_kernel(
    const XT *__restrict__ x, const float *__restrict__ wg,
    const float *__restrict__ bg, int T, int d, int E, int k, int gate,
    int32_t *__restrict__ topk_idx, float *__restrict__ topk_w,
    int32_t *__restrict__ counts, float *__restrict__ logits) {
  using G = LaneGeom<XT, EP, NWV>;
  constexpr int TPW = kWave / EP;          // tokens per wavefront
  constexpr int CC = G::CC;
  __shared__ u32x4_t lds[G::NB][G::CHUNK / 16];
  __shared__ int cnt[EP];
  const int lane = threadIdx.x % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int e = lane % EP;
  const int tl = wave * TPW + lane / EP;   // token within the workgroup
  const int tb = blockIdx.x * G::TPB;      // first token of the workgroup
  const int t = tb + tl;
  for (int i = threadIdx.x; i < EP; i += G::NTH) cnt[i] = 0;

  // buffer descriptors: x rows of this workgroup's tokens, all of W_g; reads
  // past either end return zeros
  const uint32_t row_x = (uint32_t)d * sizeof(XT);
  const uint32_t row_w = (uint32_t)d * 4u;
  const int64_t xrows = min(T - tb, G::TPB);
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<XT *>(x) + (int64_t)tb * d, 0, (uint32_t)(xrows * row_x), kBufWord3);
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float *>(wg), 0, (uint32_t)E * row_w, kBufWord3);
  // DMA block b of a chunk: x blocks first, then W_g blocks; lane l fills
  // LDS slot 64 b + l, the swizzled slot of some (row, column) of the
  // chunk, with that element's 16 bytes
  auto dma = [&](int ch) {
    u32x4_t *buf = lds[ch % G::NB];
    const int c0 = ch * CC;
#pragma unroll
    for (int i = 0; i < G::BPW; ++i) {
      const int b = min(wave * G::BPW + i, G::NBLK - 1);
      if (b < G::XBLK) {
        const int p = b * 64 + lane;
        const int r = p / G::XS;
        const int j = (p % G::XS) ^ (r % G::XM);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, buf + b * 64, 16,
                                                 (uint32_t)r * row_x + (uint32_t)j * 16u,
                                                 c0 * (int)sizeof(XT), 0, 0);
      } else {
        const int p = (b - G::XBLK) * 64 + lane;
        const int r = p / G::WS;
        const int j = (p % G::WS) ^ (r % G::WM);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, buf + b * 64, 16,
                                                 (uint32_t)r * row_w + (uint32_t)j * 16u,
                                                 c0 * 4, 0, 0);
      }
    }
  };

  float acc = 0.0f;
  const int nch = (d + CC - 1) / CC;
#pragma unroll
  for (int c = 0; c < G::NB - 1; ++c)
    if (c < nch) dma(c);
  for (int ch = 0; ch < nch; ++ch) {
    // chunk ch has landed (later chunks may be in flight), this wavefront's
    // reads of chunk ch-1 are done; then the workgroup barrier makes chunk
    // ch complete and frees the buffer of chunk ch-1 for chunk ch+3.  The
    // empty asm statements keep the compiler from moving LDS accesses
    // across the barrier (a fence would also wait for the DMAs in flight).
    const int ahead = min(nch - 1 - ch, G::NB - 2);
    if (ahead >= 2) __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(2 * G::BPW));
    else if (ahead == 1) __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(G::BPW));
    else __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (ch + G::NB - 1 < nch) dma(ch + G::NB - 1);
    const u32x4_t *xb = lds[ch % G::NB];
    const u32x4_t *wb = xb + G::XBLK * 64;
    const int ncol = min(CC, d - ch * CC);
    // The chain's operands, 32 columns at a time, in two register sets: the
    // LDS reads of the next 32 columns are issued before the FMAs of these,
    // so their latency hides behind the chain.
    constexpr int XR = sizeof(XT) == 2 ? 4 : 8;   // 16-byte x slots per 32 columns
    u32x4_t xs[2][XR], ws[2][8];
    auto rd = [&](int b, int c) {
#pragma unroll
      for (int i = 0; i < XR; ++i) xs[b][i] = xb[G::xslot(tl, c / (32 / XR) + i)];
#pragma unroll
      for (int i = 0; i < 8; ++i) ws[b][i] = wb[G::wslot(e, c / 4 + i)];
    };
    auto fma = [&](int b) {
      float xv[32];
      if constexpr (sizeof(XT) == 2)
        RowLoad<uint16_t>::expand(xs[b], xv);
      else
        RowLoad<float>::expand(xs[b], xv);
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) acc = __builtin_fmaf(xv[4 * i + q], __uint_as_float(ws[b][i][q]), acc);
    };
    // (ncol is a multiple of 64; the last prefetch re-reads the chunk's
    // last 32 columns and is not consumed, which keeps the loop branch-free)
    static_assert(CC % 64 == 0, "chunks of whole 64-column steps");
    rd(0, 0);
    for (int c = 0; c < ncol; c += 64) {
      rd(1, c + 32);
      fma(0);
      rd(0, min(c + 64, ncol - 32));
      fma(1);
    }
  }

  lane_select<EP, G::NTH>(acc, t, e, T, E, k, gate, bg, topk_idx, topk_w, counts, logits,
                          cnt);
}

template <typename XT, int EP, int NWV>
static hipError_t launch_route_lane(const void *x, const float *wg, const float *bg, int T,
                                    int d, int E, int k, int gate, int32_t *idx, float *w,
                                    int32_t *counts, float *logits, hipStream_t s) {
  using G = LaneGeom<XT, EP, NWV>;
  const int blocks = (T + G::TPB - 1) / G::TPB;
  route_lane_kernel<XT, EP, NWV><<<blocks, G::NTH, 0, s>>>(
      static_cast<const XT *>(x), wg, bg, T, d, E, k, gate, idx, w, counts, logits);
  return hipGetLastError();
}

template <typename XT, int EP>
static hipError_t launch_route_direct(const void *x, const float *wg, const float *bg,
                                      int T, int d, int E, int k, int gate, int32_t *idx,
                                      float *w, int32_t *counts, float *logits,
                                      hipStream_t s) {
  const int64_t waves = ((int64_t)T * EP + kWave - 1) / kWave;
  if (waves < 256) {
    constexpr int TPB = kWave / EP;   // tokens per one-wave workgroup
    const int blocks = (T + TPB - 1) / TPB;
    route_direct_kernel<XT, EP, kWave><<<blocks, kWave, 0, s>>>(
        static_cast<const XT *>(x), wg, bg, T, d, E, k, gate, idx, w, counts, logits);
  } else {
    constexpr int TPB = (kRouteThreads / kWave) * (kWave / EP);
    const int blocks = (T + TPB - 1) / TPB;
    route_direct_kernel<XT, EP, kRouteThreads><<<blocks, kRouteThreads, 0, s>>>(
        static_cast<const XT *>(x), wg, bg, T, d, E, k, gate, idx, w, counts, logits);
  }
  return hipGetLastError();
}

template <typename XT, int TX, int EPT, int TPT, int GMAX, int NTH = kRouteThreads>
static hipError_t launch_route_t(const void *x, const float *wg, const float *bg,
                                 int T, int d, int E, int k, int gate, int32_t *idx,
                                 float *w, int32_t *counts, float *logits,
                                 hipStream_t s) {
  constexpr int BT = (NTH / TX) * TPT;
  constexpr int CHUNK = (BT + TX * EPT) * (kRouteBK + 4);
  constexpr int EPS = TX * EPT + 1;
  // chunks per super-chunk: the most that divide d and keep the two LDS
  // buffers within 128 KB
  int G = 1;
  for (int g = GMAX; g >= 1; --g)
    if (d % (kRouteBK * g) == 0 && 2 * g * CHUNK * 4 <= 128 * 1024) {
      G = g;
      break;
    }
  size_t lds = sizeof(float) * 2 * (size_t)G * CHUNK;
  // scores (and the unbiased ones for the bias-selects gate) reuse the space
  const size_t score_lds = sizeof(float) * (size_t)BT * EPS * (gate == kGateBiasSelects ? 2 : 1);
  if (lds < score_lds) lds = score_lds;
  auto kern = route_kernel<XT, TX, EPT, TPT, GMAX, NTH>;
  hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (err != hipSuccess) return err;
  const int blocks = (T + BT - 1) / BT;
  kern<<<blocks, NTH, lds, s>>>(static_cast<const XT *>(x), wg, bg, T, d, E, k, gate, G,
                                          idx, w, counts, logits);
  return hipGetLastError();
}

// Small batches (decode): one chain per thread and a few tokens per
// workgroup, so the sequential chains spread over as many SIMDs as there
// are (token, expert) pairs; large batches: register tiles of 4 tokens.
template <typename XT>
static hipError_t launch_route_dt(const void *x, const float *wg, const float *bg,
                                  int T, int d, int E, int k, int gate, int32_t *idx,
                                  float *w, int32_t *counts, float *logits,
                                  hipStream_t s) {
  // Up to 64 experts, one chain per lane.  Batches that give at least 64
  // workgroups: operands staged in LDS (route_lane_kernel); smaller batches
  // (decode): operands streamed straight into registers by few-wavefront
  // workgroups spread over the CUs (route_direct_kernel, whose 32-bit
  // buffer offsets cover the whole of x); up to 256 tokens, one token per
  // wavefront whatever E is (lanes past E idle), so a wavefront's x loads
  // all hit one row (gpt-oss-20b decode shape: 23 us against 28 us with two
  // tokens per wavefront).  Measured on MI355X.
  const bool fits = (int64_t)T * d * (int64_t)sizeof(XT) < (int64_t(1) << 31);
#define MOE_LANE(EP)                                                                 \
  do {                                                                               \
    if (T >= 64 * LaneGeom<XT, EP, 4>::TPB || !fits)                                 \
      return launch_route_lane<XT, EP, 4>(x, wg, bg, T, d, E, k, gate, idx, w, counts, logits, s); \
    if (T <= 256)                                                                    \
      return launch_route_direct<XT, 64>(x, wg, bg, T, d, E, k, gate, idx, w, counts, logits, s); \
    return launch_route_direct<XT, EP>(x, wg, bg, T, d, E, k, gate, idx, w, counts, logits, s);   \
  } while (0)
  if (E <= 8) MOE_LANE(8);
  if (E <= 16) MOE_LANE(16);
  if (E <= 32) MOE_LANE(32);
  if (E <= 64) MOE_LANE(64);
#undef MOE_LANE
#define MOE_ROUTE(TX, EPT, TPT, GM, NTH) \
  return launch_route_t<XT, TX, EPT, TPT, GM, NTH>(x, wg, bg, T, d, E, k, gate, idx, w, counts, logits, s)
  if (E <= 128) MOE_ROUTE(32, 4, 4, 1, kRouteThreads);
  // Every workgroup streams all of W_g through LDS, so fewer, larger
  // workgroups move less of it from L2: 32 tokens in 8 wavefronts (one
  // workgroup per CU at T = 8192) once there are at least 256 of them
  // (measured on MI355X at E = 256, d = 7168: 520 us against 571 us for
  // 16 tokens in 4 wavefronts, two per CU; 32 tokens in 4 wavefronts,
  // one wavefront per SIMD, measured 726 us against 559 us)
  if (T >= 32 * 256) MOE_ROUTE(64, 4, 4, 1, 512);
  MOE_ROUTE(64, 4, 4, 1, kRouteThreads);
#undef MOE_ROUTE
}

hipError_t launch_fill_i32(int32_t *p, int n, int32_t v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int blocks = (n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024;
  fill_i32_kernel<<<blocks, 256, 0, s>>>(p, n, v);
  return hipGetLastError();
}

// counts are zeroed here, then accumulated by the route kernel; counts
// NULL: no counts (the caller takes them from the grouping)
hipError_t launch_route(bool bf16, int gate, const void *x, const float *wg,
                        const float *bg, int T, int d, int E, int k,
                        int32_t *idx, float *w, int32_t *counts, float *logits,
                        hipStream_t s) {
  hipError_t err = counts ? launch_fill_i32(counts, E, 0, s) : hipSuccess;
  if (err != hipSuccess || T == 0) return err;
  return bf16 ? launch_route_dt<uint16_t>(x, wg, bg, T, d, E, k, gate, idx, w, counts, logits, s)
              : launch_route_dt<float>(x, wg, bg, T, d, E, k, gate, idx, w, counts, logits, s);
}

}  // namespace moe
