// permute.hip - dispatch: stable grouping of the T*k assignments by expert.
//
// The "Expert Backend" section of "Understanding MoE in Transformers"
// describes the grouped backend as: sort and group the tokens by expert id,
// run one grouped GEMM, then collect and reorder.  Here the sort is a
// counting sort, stable in the flat assignment index f = t*k + j:
//   1. hist    - one workgroup per segment of kSeg assignments builds an LDS
//                histogram of expert ids (integer atomics: order-free).
//   2. scan    - one workgroup: per expert, exclusive prefix over segments,
//                counts, exclusive prefix over experts = group offsets, and
//                the first grouped row of every (segment, expert).
//   3. scatter - one workgroup per segment, one wavefront per quarter of
//                it; inside a wavefront, lanes holding the same expert are
//                matched with 8 ballots (expert ids < 256) and ranked by
//                lane order, so rows keep flat-index order.
//   4. stats   - Importance(X)_e = sum of the router weights of group e,
//                one wavefront per expert: lane l adds rows l, l+64, ...
//                of the group in order, then a fixed xor butterfly over the
//                64 partial sums (a fixed order, so deterministic; Qiita
//                summary "Load-balancing losses"); then one wavefront computes
//                CV^2(Importance), CV^2(Load) and the load-balance loss of
//                the Go chapter's section 3, in fp64.
//   5. move    - x_perm[p] = x[perm_src[p]], 16-byte vectors, one row per
//                workgroup iteration (coalesced reads and writes).
//
// Expert capacity C (the Go chapter's "What was simplified": an expert
// accepts a bounded number of tokens and the overflow is dropped): an
// assignment whose rank within its expert's group (flat order) is C or more
// is dropped.  Kept assignments get compacted rows (offsets over the kept
// rows, pos = -1 for a dropped one); Importance and the statistics keep the
// router's view (every assignment), through the full group starts.
#include "common.h"
#include "permute.h"

#include <mutex>

namespace moe {

constexpr int kSeg = 1024;          // assignments per segment
constexpr int kPermThreads = 256;   // 4 wavefronts x 256 assignments

__global__ __launch_bounds__(kPermThreads) void perm_hist_kernel(
    const int32_t *__restrict__ idx, int n, int E, int32_t *__restrict__ hist) {
  __shared__ int h[kMaxExperts];
  for (int e = threadIdx.x; e < E; e += kPermThreads) h[e] = 0;
  __syncthreads();
  const int f0 = blockIdx.x * kSeg;
  const int f1 = min(n, f0 + kSeg);
  for (int f = f0 + threadIdx.x; f < f1; f += kPermThreads) {
    const int e = idx[f];
    if (static_cast<unsigned>(e) < static_cast<unsigned>(E)) atomicAdd(&h[e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kPermThreads)
    hist[(int64_t)blockIdx.x * E + e] = h[e];
}

// One workgroup of 256 threads; thread e owns expert e.  full_off: group
// starts over every assignment; offsets: over the kept ones (capacity cap).
__global__ __launch_bounds__(kPermThreads) void perm_scan_kernel(
    int32_t *__restrict__ hist, int nseg, int E, int n, int cap,
    int32_t *__restrict__ full_off, int32_t *__restrict__ offsets,
    int32_t *__restrict__ counts_out) {
  __shared__ int sc[kPermThreads], kc[kPermThreads];
  const int e = threadIdx.x;
  int total = 0;
  if (e < E) {
    for (int s = 0; s < nseg; ++s) {
      const int c = hist[(int64_t)s * E + e];
      hist[(int64_t)s * E + e] = total;
      total += c;
    }
  }
  sc[e] = total;
  kc[e] = min(total, cap);
  __syncthreads();
  // inclusive Hillis-Steele scans over the 256 expert totals
  for (int off = 1; off < kPermThreads; off <<= 1) {
    const int v = e >= off ? sc[e - off] : 0;
    const int u = e >= off ? kc[e - off] : 0;
    __syncthreads();
    sc[e] += v;
    kc[e] += u;
    __syncthreads();
  }
  const int start = sc[e] - total;  // exclusive
  if (e < E) {
    if (counts_out) counts_out[e] = total;
    full_off[e] = start;
    offsets[e] = kc[e] - min(total, cap);
    for (int s = 0; s < nseg; ++s) hist[(int64_t)s * E + e] += start;
  }
  if (e == 0) {
    full_off[E] = n;
    offsets[E] = kc[kPermThreads - 1];
  }
}

__global__ __launch_bounds__(kPermThreads) void perm_scatter_kernel(
    const int32_t *__restrict__ idx, const float *__restrict__ w, int n, int k,
    int E, int cap, const int32_t *__restrict__ base,
    const int32_t *__restrict__ full_off, const int32_t *__restrict__ offsets,
    int32_t *__restrict__ pos, int32_t *__restrict__ perm_src,
    float *__restrict__ perm_w) {
  constexpr int NW = kPermThreads / kWave;
  constexpr int SUB = kSeg / NW;    // assignments per wavefront
  __shared__ int run[NW][kMaxExperts];
  const int lane = threadIdx.x % kWave;
  const int wv = threadIdx.x / kWave;
  const int f0 = blockIdx.x * kSeg + wv * SUB;

  for (int i = threadIdx.x; i < NW * kMaxExperts; i += kPermThreads) (&run[0][0])[i] = 0;
  __syncthreads();
  for (int c = 0; c < SUB; c += kWave) {
    const int f = f0 + c + lane;
    if (f < n) {
      const int e = idx[f];
      if (static_cast<unsigned>(e) < static_cast<unsigned>(E)) atomicAdd(&run[wv][e], 1);
    }
  }
  __syncthreads();
  // per-wavefront first grouped row of every expert
  for (int e = threadIdx.x; e < E; e += kPermThreads) {
    int r = base[(int64_t)blockIdx.x * E + e];
    for (int v = 0; v < NW; ++v) {
      const int c = run[v][e];
      run[v][e] = r;
      r += c;
    }
  }
  __syncthreads();
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int c = 0; c < SUB; c += kWave) {
    const int f = f0 + c + lane;
    int e = f < n ? idx[f] : -1;
    const bool valid = static_cast<unsigned>(e) < static_cast<unsigned>(E);
    if (!valid) e = 0;
    uint64_t peers = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t m = __ballot(valid && bit);
      peers &= bit ? m : ~m;
    }
    if (valid) {
      const int rank = __popcll(peers & below);
      const int p = run[wv][e] + rank;
      const int r = p - full_off[e];   // rank within the expert's group
      perm_w[p] = w[f];
      if (r < cap) {
        const int q = offsets[e] + r;
        pos[f] = q;
        perm_src[q] = f / k;
      } else {
        pos[f] = -1;
      }
      // the lowest lane of each peer group advances the group's next row;
      // every lane read run[] above, before this store (in-order LDS)
      if (rank == 0) run[wv][e] = p + __popcll(peers);
    }
  }
}

// importance[e]: one wavefront per expert sums the router weights of its
// group (every assignment, starts `full_off`; lane-strided partial sums,
// then a fixed butterfly: deterministic).
__global__ __launch_bounds__(kPermThreads) void perm_importance_kernel(
    const int32_t *__restrict__ offsets, const float *__restrict__ perm_w,
    int E, float *__restrict__ importance) {
  const int lane = threadIdx.x % kWave;
  const int e = blockIdx.x * (kPermThreads / kWave) + threadIdx.x / kWave;
  if (e >= E) return;
  const int r0 = offsets[e], r1 = offsets[e + 1];
  float s = 0.0f;
  for (int r = r0 + lane; r < r1; r += kWave) s += perm_w[r];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
  if (lane == 0) importance[e] = s;
}

// One wavefront: CV^2(Importance), CV^2(Load) and the load-balance loss, in
// fp64 with a fixed reduction order.
__global__ __launch_bounds__(kWave) void perm_stats_kernel(
    const int32_t *__restrict__ offsets, const float *__restrict__ importance,
    int E, double *__restrict__ stats) {
  const int lane = threadIdx.x;
  double si = 0.0, sc = 0.0;
  for (int e = lane; e < E; e += kWave) {
    si += importance[e];
    sc += offsets[e + 1] - offsets[e];
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    si += __shfl_xor(si, off);
    sc += __shfl_xor(sc, off);
  }
  const double mi = si / E, mc = sc / E;
  double vi = 0.0, vc = 0.0, f2 = 0.0;
  for (int e = lane; e < E; e += kWave) {
    const double c = offsets[e + 1] - offsets[e];
    const double im = importance[e];
    vi += (im - mi) * (im - mi);
    vc += (c - mc) * (c - mc);
    if (sc != 0.0) f2 += (c / sc) * (c / sc);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    vi += __shfl_xor(vi, off);
    vc += __shfl_xor(vc, off);
    f2 += __shfl_xor(f2, off);
  }
  if (lane == 0) {
    stats[0] = mi == 0.0 ? 0.0 : (vi / E) / (mi * mi);
    stats[1] = mc == 0.0 ? 0.0 : (vc / E) / (mc * mc);
    stats[2] = sc == 0.0 ? 0.0 : E * f2;
  }
}

// x_perm[p] = x[perm_src[p]] for the kept rows p < *kept_rows; row_vec16 =
// bytes per row / 16.  The source index is clamped to [0, T) so that a
// corrupt index cannot read outside x.
__global__ __launch_bounds__(kPermThreads) void perm_move_kernel(
    const uint4 *__restrict__ x, const int32_t *__restrict__ perm_src,
    const int32_t *__restrict__ kept_rows, int n, int T, int row_vec16,
    uint4 *__restrict__ x_perm) {
  const int rows = min(max(*kept_rows, 0), n);
  for (int p = blockIdx.x; p < rows; p += gridDim.x) {
    const int t = min(max(perm_src[p], 0), T - 1);
    const uint4 *src = x + (int64_t)t * row_vec16;
    uint4 *dst = x_perm + (int64_t)p * row_vec16;
    for (int i = threadIdx.x; i < row_vec16; i += kPermThreads) dst[i] = src[i];
  }
}

// Steps 1-4 in one workgroup for up to kFusedMax assignments (decode and
// small prefill batches), where launch latency outweighs the work (measured:
// 7 us for 256 assignments against about 22 us for the five launches, break
// even near 6000).  Same arithmetic as the multi-workgroup kernels: the stable
// order (flat index, ballot ranks within a wavefront, wavefront order within
// a chunk, chunk order), the Importance sums and the statistics are
// computed in the same order, so both paths give identical results.
constexpr int kFusedThreads = 1024;
constexpr int kFusedMax = 4096;

__global__ __launch_bounds__(kFusedThreads) void perm_fused_kernel(
    const int32_t *__restrict__ idx, const float *__restrict__ w, int n, int k,
    int E, int cap, int32_t *__restrict__ offsets, int32_t *__restrict__ pos,
    int32_t *__restrict__ perm_src, float *__restrict__ perm_w,
    float *__restrict__ importance, double *__restrict__ stats,
    int32_t *__restrict__ counts_out) {
  constexpr int NW = kFusedThreads / kWave;
  __shared__ int h[kMaxExperts];
  __shared__ int off[kMaxExperts + 1];    // full group starts
  __shared__ int koff[kMaxExperts];       // kept group starts
  __shared__ int run[NW][kMaxExperts];
  __shared__ int scan_tmp[NW];
  __shared__ float pw[kFusedMax];         // the weights in grouped order
  constexpr int NC = kFusedMax / kFusedThreads;
  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wv = tid / kWave;

  // every assignment's expert and weight, loaded once up front (thread tid
  // holds assignments tid + c * kFusedThreads)
  int ea[NC];
  float wa[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int f = tid + c * kFusedThreads;
    ea[c] = f < n ? idx[f] : -1;
    wa[c] = f < n ? w[f] : 0.0f;
  }
  // 1. histogram
  for (int e = tid; e < kMaxExperts; e += kFusedThreads) h[e] = 0;
  __syncthreads();
#pragma unroll
  for (int c = 0; c < NC; ++c)
    if (static_cast<unsigned>(ea[c]) < static_cast<unsigned>(E)) atomicAdd(&h[ea[c]], 1);
  __syncthreads();
  // 2. group offsets: exclusive scans over the experts, of every assignment
  //    (full) and of the kept ones (capacity)
  {
    const int c = tid < E ? h[tid] : 0;
    int total, ktotal;
    const int ex = block_exclusive_scan<kFusedThreads>(c, scan_tmp, &total);
    const int kex = block_exclusive_scan<kFusedThreads>(min(c, cap), scan_tmp, &ktotal);
    if (tid < E) {
      if (counts_out) counts_out[tid] = c;
      off[tid] = ex;
      koff[tid] = kex;
      offsets[tid] = kex;
      h[tid] = ex;          // running first full row of each expert
    }
    if (tid == 0) {
      off[E] = n;
      offsets[E] = ktotal;
    }
  }
  __syncthreads();
  // 3. stable scatter, one chunk of kFusedThreads assignments at a time
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int c0 = c * kFusedThreads;
    if (c0 >= n) break;
    const int f = c0 + tid;
    int e = ea[c];
    const bool valid = static_cast<unsigned>(e) < static_cast<unsigned>(E);
    if (!valid) e = 0;
    uint64_t peers = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t m = __ballot(valid && bit);
      peers &= bit ? m : ~m;
    }
    const int rank = __popcll(peers & below);
    for (int i = tid; i < NW * kMaxExperts; i += kFusedThreads) (&run[0][0])[i] = 0;
    __syncthreads();
    if (valid && rank == 0) run[wv][e] = __popcll(peers);
    __syncthreads();
    for (int x = tid; x < E; x += kFusedThreads) {
      int r = h[x];
      for (int v = 0; v < NW; ++v) {
        const int cnt = run[v][x];
        run[v][x] = r;
        r += cnt;
      }
      h[x] = r;
    }
    __syncthreads();
    if (valid) {
      const int p = run[wv][e] + rank;
      const int r = p - off[e];
      perm_w[p] = wa[c];
      pw[p] = wa[c];
      if (r < cap) {
        const int q = koff[e] + r;
        pos[f] = q;
        perm_src[q] = f / k;
      } else {
        pos[f] = -1;
      }
    }
    __syncthreads();
  }
  // 4. Importance, one wavefront per expert (lane-strided sums, butterfly)
  __shared__ float imp[kMaxExperts];
  for (int x = wv; x < E; x += NW) {
    float sum = 0.0f;
    for (int r = off[x] + lane; r < off[x + 1]; r += kWave) sum += pw[r];
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) sum += __shfl_xor(sum, o);
    if (lane == 0) {
      if (importance) importance[x] = sum;
      imp[x] = sum;
    }
  }
  __syncthreads();
  if (!stats || wv != 0) return;
  // statistics: the fp64 reductions of perm_stats_kernel
  double si = 0.0, sc = 0.0;
  for (int x = lane; x < E; x += kWave) {
    si += imp[x];
    sc += off[x + 1] - off[x];
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    si += __shfl_xor(si, o);
    sc += __shfl_xor(sc, o);
  }
  const double mi = si / E, mc = sc / E;
  double vi = 0.0, vc = 0.0, f2 = 0.0;
  for (int x = lane; x < E; x += kWave) {
    const double cnt = off[x + 1] - off[x];
    const double im = imp[x];
    vi += (im - mi) * (im - mi);
    vc += (cnt - mc) * (cnt - mc);
    if (sc != 0.0) f2 += (cnt / sc) * (cnt / sc);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    vi += __shfl_xor(vi, o);
    vc += __shfl_xor(vc, o);
    f2 += __shfl_xor(f2, o);
  }
  if (lane == 0) {
    stats[0] = mi == 0.0 ? 0.0 : (vi / E) / (mi * mi);
    stats[1] = mc == 0.0 ? 0.0 : (vc / E) / (mc * mc);
    stats[2] = sc == 0.0 ? 0.0 : E * f2;
  }
}

// Next-choice re-routing of the capacity overflow (Go chapter, "Design
// viewpoints": an overflowing token is dropped or handed to its next
// candidate), one hop: the o-th overflowing slot of a token (slot order) is
// offered to its o-th best expert outside its top k (higher score first,
// ties to the lower index), and each expert accepts offers in flat order
// into the room the first round left.  Three groupings run in stream order:
// the drop rule on the top k (which also gives Importance and the
// statistics, the router's view), the offers (ranks among the offers to each
// expert), and the final one over the computing expert of every slot.

// One wavefront per token: cand[f] = the expert offered to overflowing slot
// f, -1 for a kept slot or when the token has no expert left to offer.
__global__ __launch_bounds__(kWave) void reroute_offer_kernel(
    const int32_t *__restrict__ idx, const int32_t *__restrict__ pos_a,
    const float *__restrict__ logits, int k, int E, int32_t *__restrict__ cand) {
  constexpr int Q = kMaxExperts / kWave;
  const int t = blockIdx.x;
  const int lane = threadIdx.x;
  const int32_t *it = idx + (int64_t)t * k;
  const int32_t *pa = pos_a + (int64_t)t * k;
  int32_t *ct = cand + (int64_t)t * k;
  int nover = 0;
  for (int j = 0; j < k; ++j) nover += pa[j] < 0;
  if (nover == 0) {
    for (int j = lane; j < k; j += kWave) ct[j] = -1;
    return;
  }
  float sc[Q];
  bool avail[Q];
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const int e = lane + kWave * q;
    bool a = e < E;
    for (int j = 0; j < k && a; ++j) a = it[j] != e;
    avail[q] = a;
    sc[q] = a ? logits[(int64_t)t * E + e] : 0.0f;
  }
  for (int j = 0; j < k; ++j) {   // uniform over the wavefront
    if (pa[j] >= 0) {
      if (lane == 0) ct[j] = -1;
      continue;
    }
    // best available (score descending, index ascending)
    bool ba = false;
    float bs = 0.0f;
    int be = 0x7fffffff;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int e = lane + kWave * q;
      if (avail[q] && (!ba || sc[q] > bs || (sc[q] == bs && e < be))) {
        ba = true;
        bs = sc[q];
        be = e;
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const bool oa = __shfl_xor((int)ba, off) != 0;
      const float os = __shfl_xor(bs, off);
      const int oe = __shfl_xor(be, off);
      if (oa && (!ba || os > bs || (os == bs && oe < be))) {
        ba = true;
        bs = os;
        be = oe;
      }
    }
    if (lane == 0) ct[j] = ba ? be : -1;
    if (ba && (be % kWave) == lane) avail[be / kWave] = false;
  }
}

// fin[f]: the expert that computes slot f after both rounds, -1 if dropped;
// pos[f] = -1 (the final grouping writes the computed slots' rows).
__global__ void reroute_accept_kernel(
    const int32_t *__restrict__ idx, const int32_t *__restrict__ pos_a,
    const int32_t *__restrict__ cand, const int32_t *__restrict__ pos_b,
    const int32_t *__restrict__ kept_a, const int32_t *__restrict__ off_b, int n, int E,
    int cap, int32_t *__restrict__ fin, int32_t *__restrict__ pos) {
  const int f = blockIdx.x * blockDim.x + threadIdx.x;
  if (f >= n) return;
  int out = -1;
  if (pos_a[f] >= 0) {
    out = idx[f];
  } else {
    const int e = cand[f];
    if (static_cast<unsigned>(e) < static_cast<unsigned>(E)) {
      const int room = cap - (kept_a[e + 1] - kept_a[e]);   // first-round starts
      if (pos_b[f] - off_b[e] < room) out = e;
    }
  }
  fin[f] = out;
  pos[f] = -1;
}

__global__ void zero_f32_kernel(float *p, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0.0f;
}
__global__ void zero_stats_kernel(double *p) {
  if (threadIdx.x < 3) p[threadIdx.x] = 0.0;
}

hipError_t launch_zero_stats(float *importance, int E, double *stats, hipStream_t s) {
  if (importance) zero_f32_kernel<<<1, 256, 0, s>>>(importance, E);
  if (stats) zero_stats_kernel<<<1, 64, 0, s>>>(stats);
  return hipGetLastError();
}

int perm_num_segments(int64_t n) { return static_cast<int>((n + kSeg - 1) / kSeg); }

// Workspace: hist [nseg * E] int32, full_off [E + 1] int32, perm_w [n] fp32.
hipError_t launch_permute(const int32_t *idx, const float *w, const void *x,
                          int T, int k, int E, int capacity, int row_bytes,
                          int32_t *offsets, int32_t *perm_src, int32_t *pos,
                          float *importance, double *stats, void *x_perm,
                          int32_t *hist, int32_t *full_off, float *perm_w,
                          hipStream_t s, int32_t *counts_out) {
  const int n = T * k;
  if (n == 0) return launch_zero_stats(importance, E, stats, s);
  const int cap = capacity > 0 ? capacity : n;
  const int blocks = n < 8192 ? n : 8192;
  if (n <= kFusedMax) {
    perm_fused_kernel<<<1, kFusedThreads, 0, s>>>(idx, w, n, k, E, cap, offsets, pos,
                                                  perm_src, perm_w, importance, stats,
                                                  counts_out);
  } else {
    const int nseg = perm_num_segments(n);
    perm_hist_kernel<<<nseg, kPermThreads, 0, s>>>(idx, n, E, hist);
    perm_scan_kernel<<<1, kPermThreads, 0, s>>>(hist, nseg, E, n, cap, full_off, offsets,
                                                counts_out);
    perm_scatter_kernel<<<nseg, kPermThreads, 0, s>>>(idx, w, n, k, E, cap, hist, full_off,
                                                      offsets, pos, perm_src, perm_w);
    if (importance) {   // NULL: grouping only
      perm_importance_kernel<<<(E + 3) / 4, kPermThreads, 0, s>>>(full_off, perm_w, E,
                                                                  importance);
      if (stats) perm_stats_kernel<<<1, kWave, 0, s>>>(full_off, importance, E, stats);
    }
  }
  if (x_perm)   // NULL: grouping only (the backward pass regroups every assignment)
    perm_move_kernel<<<blocks, kPermThreads, 0, s>>>(
        static_cast<const uint4 *>(x), perm_src, offsets + E, n, T, row_bytes / 16,
        static_cast<uint4 *>(x_perm));
  return hipGetLastError();
}

hipError_t launch_permute_reroute(const int32_t *idx, const float *w, const float *logits,
                                  const void *x, int T, int k, int E, int capacity,
                                  int row_bytes, int32_t *offsets, int32_t *perm_src,
                                  int32_t *pos, float *importance, double *stats,
                                  void *x_perm, int32_t *hist, int32_t *full_off,
                                  float *perm_w, const RerouteScratch &r, hipStream_t s,
                                  int32_t *counts_out) {
  const int n = T * k;
  if (n == 0) return launch_zero_stats(importance, E, stats, s);
  hipError_t err;
  // 1. the drop rule on the top k: kept slots, Importance, statistics
  if ((err = launch_permute(idx, w, nullptr, T, k, E, capacity, row_bytes, offsets, perm_src,
                            r.pos_a, importance, stats, nullptr, hist, full_off, perm_w, s,
                            counts_out)) != hipSuccess)
    return err;
  // 2. offers, and their ranks within each expert's offers (flat order)
  reroute_offer_kernel<<<T, kWave, 0, s>>>(idx, r.pos_a, logits, k, E, r.cand);
  if ((err = launch_permute(r.cand, w, nullptr, T, k, E, 0, row_bytes, r.off_b, perm_src,
                            r.pos_b, nullptr, nullptr, nullptr, hist, r.full_off_b, perm_w,
                            s)) != hipSuccess)
    return err;
  // (offsets still holds the first round's kept group starts here)
  reroute_accept_kernel<<<(n + 255) / 256, 256, 0, s>>>(idx, r.pos_a, r.cand, r.pos_b, offsets,
                                                        r.off_b, n, E, capacity, r.fin, pos);
  // 3. the grouping by computing expert, with the row move
  return launch_permute(r.fin, w, x, T, k, E, 0, row_bytes, offsets, perm_src, pos, nullptr,
                        nullptr, x_perm, hist, r.full_off_b, perm_w, s);
}

// Scratch of the allocation-free dispatch (moe_permute_noalloc): one array
// per GPU in the code object, held until the process ends.  Host code never
// uses the array's name as an address (it is a host-side stand-in): the
// device address is taken once per device with hipGetSymbolAddress and kept.
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

hipError_t noalloc_scratch(void **ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void *addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

}  // namespace moe
