// gemm_bf16.hip - grouped GEMM of the expert FFNs on bf16 MFMA (gfx950).
//
// Only the experts a token selected are computed (conditional computation:
// the Qiita summary of "Sparsely-Gated MoE", section "Sparsely-Gated MoE
// layer formula"), so the work is a GEMM per expert over that expert's rows
// of the grouped activations: the "grouped_mm" backend of "Understanding MoE
// in Transformers" ("Expert Backend"), written here for CDNA4.
//
//   up   : hidden[r, n] = act( sum_i A[r, i] * W[e][n, i] )   (+ bias, GELU)
//          SwiGLU: act = silu(gate row n) * (up row h + n) of W = [2h, d]
//   down : y_perm[r, c] = sum_n hidden[r, n] * W2[e][c, n]     (+ bias)
//
// Both operands are K-contiguous, so tiles of either are rows of 128 B
// (BK = 64 bf16).  The MFMA is v_mfma_f32_16x16x32_bf16 with the weight rows
// as its A operand (M side) and the token rows as its B operand (N side):
// a lane then owns 4 consecutive output columns of one token row, and the
// epilogue stores 8-byte runs.  fp32 accumulation in registers.
//
// Tiles: BM token rows x BNW weight rows x BK.  Global -> registers -> LDS,
// double-buffered (one barrier per K step); 16-byte LDS chunks are XOR-
// swizzled per row so the fragment reads of 16 consecutive rows hit
// distinct banks.  A persistent grid walks the ragged tile space: every
// workgroup computes the per-group tile prefix from the group offsets, then
// takes tiles in a slice order that keeps each XCD (workgroups are dealt to
// the 8 XCDs round-robin) on a contiguous run of tiles, i.e. the m-tiles of
// a few neighbouring weight tiles, so weight tiles are fetched from HBM once
// per XCD and reused from its L2.
#include "common.h"

namespace moe {

enum GemmMode { kUpGelu = 0, kUpSwiglu = 1, kDown = 2 };

struct GemmArgs {
  const int32_t *offsets;   // [E + 1]
  int E, S, T, routed_rows; // routed_rows = T * k
  const uint16_t *a_routed; // grouped rows, [routed_rows, K]
  const uint16_t *a_shared; // shared-expert rows, [T, K] (S = 1)
  int K;
  const uint16_t *w;        // [E, w_rows, K]
  const uint16_t *w_shared; // [1, w_rows, K]
  int w_rows;               // h (GELU up), 2h (SwiGLU up), d (down)
  const uint16_t *bias;     // [E, n_out] or NULL
  uint16_t *c;              // [routed_rows + S*T, n_out]
  int n_out;                // h (up) or d (down)
  int n_tiles;              // ceil(n_out / BN_out)
  int min_rows, max_rows;   // this launch takes the groups whose row count
                            // lies in [min_rows, max_rows]
};

// Word 3 of a raw buffer resource on gfx9-family parts (32-bit data format,
// no swizzle, no index stride).
constexpr int kBufferWord3 = 0x00020000;

// LDS placement of 16-byte chunk `chunk` of tile row `row`.  With 32-wide
// k stages a row is 64 B and a fragment read (16 rows x 4 chunks) is one
// contiguous 1 KB block: no swizzle.  With 64-wide stages the 128-B rows are
// XOR-swizzled (pattern chosen by measuring fragment-read throughput).
template <int BK>
__device__ __forceinline__ int swz(int chunk, int row) {
  if constexpr (BK == 32) return chunk;
  return chunk ^ ((((row >> 2) & 3) << 1) ^ ((row >> 1) & 1));
}

// At least two waves per SIMD: 8-wave tiles run one workgroup per CU,
// 4-wave tiles two (their register budget is capped at 256 per lane).
template <int BM, int BNW, int WM, int WN, int BK, int PFD, int MODE>
__global__ __launch_bounds__(WM *WN * 64) __attribute__((amdgpu_waves_per_eu(2)))
void gemm_bf16_kernel(GemmArgs a) {
  constexpr int NT = WM * WN * 64;
  constexpr int CH = BK / 8;             // 16-byte chunks per row
  constexpr int KS = BK / 32;            // k32 MFMA steps per stage
  constexpr int WTM = BM / WM;           // token rows per wave
  constexpr int WTW = BNW / WN;          // weight rows per wave
  constexpr int FM = WTM / 16;
  constexpr int FW = WTW / 16;
  constexpr bool SWI = MODE == kUpSwiglu;
  constexpr int BN_OUT = SWI ? BNW / 2 : BNW;
  constexpr int A_LD = BM * CH / NT;     // 16-byte loads per thread per stage
  constexpr int W_LD = BNW * CH / NT;
  static_assert(BK == 32 || BK == 64, "stage depth");
  static_assert(FM >= 1 && FW >= 1 && (!SWI || FW % 2 == 0), "wave tile");
  static_assert(A_LD * NT == BM * CH && W_LD * NT == BNW * CH, "load split");
  static_assert(!SWI || (W_LD % 2 == 0), "gate and up rows split the loads evenly");

  __shared__ u32x4_t As[2][BM * CH];
  __shared__ u32x4_t Ws[2][BNW * CH];
  __shared__ int tprefix[2 * NT + 2];
  __shared__ int scan_tmp[NT / 64];
  static_assert(2 * NT >= kMaxExperts + 1, "two groups per thread cover E + S");

  const int tid = threadIdx.x;
  const int lane = tid % 64;
  const int wave = tid / 64;
  const int wm = wave / WN;
  const int wn = wave % WN;
  const int G = a.E + a.S;

  // ---- per-group m-tile prefix (exclusive), safe against bad offsets.
  // Thread t owns groups 2t and 2t+1 (G <= 257 <= 2 * NT). ----
  {
    int c2[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int g = 2 * tid + q;
      int rows = 0;
      if (g < a.E) {
        const int r0 = min(max(a.offsets[g], 0), a.routed_rows);
        const int r1 = min(max(a.offsets[g + 1], r0), a.routed_rows);
        rows = r1 - r0;
      } else if (g < G) {
        rows = a.T;
      }
      if (rows < a.min_rows || rows > a.max_rows) rows = 0;
      c2[q] = (rows + BM - 1) / BM;
    }
    int total;
    const int ex = block_exclusive_scan<NT>(c2[0] + c2[1], scan_tmp, &total);
    if (2 * tid < G + 1) tprefix[2 * tid] = ex;
    if (2 * tid + 1 < G + 1) tprefix[2 * tid + 1] = ex + c2[0];
    if (tid == 0) tprefix[G] = total;
  }
  __syncthreads();
  const int total_tiles = tprefix[G] * a.n_tiles;
  const int nk = a.K / BK;
  const int lrow = lane % 16;
  const int lch = lane / 16;

  const int nblk = gridDim.x;
  for (int it = 0;; ++it) {
    // slice order: XCD x (= blockIdx % 8) takes a contiguous run of tiles
    const int L = it * nblk + (blockIdx.x % 8) * (nblk / 8) + blockIdx.x / 8;
    if (L >= total_tiles) break;
    // group g owns tiles [tprefix[g] * n_tiles, tprefix[g+1] * n_tiles)
    int lo = 0, hi = G - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) / 2;
      if (tprefix[mid] * a.n_tiles <= L) lo = mid; else hi = mid - 1;
    }
    // tile coordinates are workgroup-uniform: make that explicit so group
    // bases and buffer descriptors live in scalar registers
    const int g = __builtin_amdgcn_readfirstlane(lo);
    const int tpg = __builtin_amdgcn_readfirstlane(tprefix[g]);
    const int tg = __builtin_amdgcn_readfirstlane(tprefix[g + 1]) - tpg;
    const int local = L - tpg * a.n_tiles;
    const int nt = local / tg;
    const int mt = local % tg;

    int grow0, rows;   // first grouped row (of c) and row count of group g
    const uint16_t *abase;
    const uint16_t *wbase;
    if (g < a.E) {
      const int r0 = min(max(a.offsets[g], 0), a.routed_rows);
      const int r1 = min(max(a.offsets[g + 1], r0), a.routed_rows);
      grow0 = r0;
      rows = r1 - r0;
      abase = a.a_routed + (int64_t)r0 * a.K;
      wbase = a.w + (int64_t)g * a.w_rows * a.K;
    } else {
      grow0 = a.routed_rows;
      rows = a.T;
      abase = a.a_shared;
      wbase = a.w_shared;
    }
    const int m0 = mt * BM;
    const int n0 = nt * BN_OUT;

    // Buffer descriptors over this tile's rows: loads past the last valid
    // row (group tail, N tail) are out of range and return zeros, so no
    // clamping is needed and one 32-bit offset per thread addresses all
    // of its 16-byte loads.
    const uint32_t row_bytes = (uint32_t)a.K * 2u;
    const int arows = min(BM, rows - m0);
    const __amdgpu_buffer_rsrc_t rs_a = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(abase + (int64_t)m0 * a.K), 0, arows * row_bytes, kBufferWord3);
    __amdgpu_buffer_rsrc_t rs_w0, rs_w1;
    if constexpr (SWI) {
      const int h = a.n_out;
      const int wv = min(BNW / 2, h - n0);
      rs_w0 = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t *>(wbase + (int64_t)n0 * a.K), 0, wv * row_bytes, kBufferWord3);
      rs_w1 = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t *>(wbase + (int64_t)(h + n0) * a.K), 0, wv * row_bytes, kBufferWord3);
    } else {
      const int wv = min(BNW, a.w_rows - n0);
      rs_w0 = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t *>(wbase + (int64_t)n0 * a.K), 0, wv * row_bytes, kBufferWord3);
      rs_w1 = rs_w0;
    }
    // thread's first row (tid / CH) and 16-byte chunk (tid % CH); load i
    // covers row tid / CH + i * (NT / CH)
    const uint32_t voff0 = (uint32_t)(tid / CH) * row_bytes + (uint32_t)(tid % CH) * 16u;
    const uint32_t istride = (uint32_t)(NT / CH) * row_bytes;

    f32x4_t acc[FW][FM];
#pragma unroll
    for (int i = 0; i < FW; ++i)
#pragma unroll
      for (int j = 0; j < FM; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // Two register stages (prefetch distance 2) feed two LDS buffers: the
    // loads of stage k+2 are issued while stage k is computed and stored to
    // LDS only after stage k+1 is computed.
    u32x4_t ra0[A_LD], rw0[W_LD];
    u32x4_t ra1[PFD == 2 ? A_LD : 1], rw1[PFD == 2 ? W_LD : 1];
    auto gload = [&](u32x4_t(&ra)[A_LD], u32x4_t(&rw)[W_LD], int kt) {
      const uint32_t ko = (uint32_t)kt * (BK * 2);
#pragma unroll
      for (int i = 0; i < A_LD; ++i)
        ra[i] = __builtin_amdgcn_raw_buffer_load_b128(rs_a, voff0 + i * istride + ko, 0, 0);
#pragma unroll
      for (int i = 0; i < W_LD; ++i) {
        if (!SWI || i < W_LD / 2) {
          rw[i] = __builtin_amdgcn_raw_buffer_load_b128(rs_w0, voff0 + i * istride + ko, 0, 0);
        } else {
          rw[i] = __builtin_amdgcn_raw_buffer_load_b128(
              rs_w1, voff0 + (i - W_LD / 2) * istride + ko, 0, 0);
        }
      }
    };
    auto lstore = [&](const u32x4_t(&ra)[A_LD], const u32x4_t(&rw)[W_LD], int buf) {
#pragma unroll
      for (int i = 0; i < A_LD; ++i) {
        const int q = tid + i * NT;
        As[buf][(q / CH) * CH + swz<BK>(q % CH, q / CH)] = ra[i];
      }
#pragma unroll
      for (int i = 0; i < W_LD; ++i) {
        const int q = tid + i * NT;
        Ws[buf][(q / CH) * CH + swz<BK>(q % CH, q / CH)] = rw[i];
      }
    };
    auto wrow = [&](int i) {
      if constexpr (SWI) {
        return (i < FW / 2) ? wn * (WTW / 2) + i * 16 + lrow
                            : BNW / 2 + wn * (WTW / 2) + (i - FW / 2) * 16 + lrow;
      } else {
        return wn * WTW + i * 16 + lrow;
      }
    };
    // Token fragments of every k32 step are read first, then weight
    // fragments are streamed PD ahead of the MFMAs that use them.
    auto compute = [&](int buf) {
      bf16x8_t fa[KS][FM], fw[KS][FW];
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const int ch = 4 * s + lch;
#pragma unroll
        for (int j = 0; j < FM; ++j) {
          const int r = wm * WTM + j * 16 + lrow;
          fa[s][j] = __builtin_bit_cast(bf16x8_t, As[buf][r * CH + swz<BK>(ch, r)]);
        }
      }
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const int ch = 4 * s + lch;
#pragma unroll
        for (int i = 0; i < FW; ++i) {
          const int r = wrow(i);
          fw[s][i] = __builtin_bit_cast(bf16x8_t, Ws[buf][r * CH + swz<BK>(ch, r)]);
        }
      }
#pragma unroll
      for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int i = 0; i < FW; ++i)
#pragma unroll
          for (int j = 0; j < FM; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fw[s][i], fa[s][j], acc[i][j], 0, 0, 0);
      constexpr int NWF = KS * FW;
      constexpr int PD = (8 + FM - 1) / FM < NWF ? (8 + FM - 1) / FM : NWF;
      __builtin_amdgcn_sched_group_barrier(0x100, KS * FM + PD, 0);
#pragma unroll
      for (int n = 0; n < NWF; ++n) {
        __builtin_amdgcn_sched_group_barrier(0x008, FM, 0);
        if (n + PD < NWF) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    };

    // Scheduling fences keep each stage's global loads ahead of the MFMAs
    // (the compiler would otherwise sink them next to their LDS stores and
    // expose the whole load latency).
    if constexpr (PFD == 2) {
      gload(ra0, rw0, 0);
      lstore(ra0, rw0, 0);
      gload(ra1, rw1, 1);
      __syncthreads();
      int kt = 0;
      for (; kt + 2 <= nk; kt += 2) {
        // even step: LDS buffer 0 holds stage kt, registers 1 hold stage kt+1
        gload(ra0, rw0, kt + 2);
        __builtin_amdgcn_sched_barrier(0);
        compute(0);
        __builtin_amdgcn_sched_barrier(0);
        lstore(ra1, rw1, 1);
        __syncthreads();
        // odd step: LDS buffer 1 holds stage kt+1, registers 0 hold stage kt+2
        gload(ra1, rw1, kt + 3);
        __builtin_amdgcn_sched_barrier(0);
        compute(1);
        __builtin_amdgcn_sched_barrier(0);
        lstore(ra0, rw0, 0);
        __syncthreads();
      }
      if (kt < nk) compute(0);   // odd stage count: the last stage is in buffer 0
    } else {
      // one register stage: the loads of stage k+1 fly while stage k computes
      gload(ra0, rw0, 0);
      lstore(ra0, rw0, 0);
      __syncthreads();
      for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        gload(ra0, rw0, kt + 1);
        __builtin_amdgcn_sched_barrier(0);
        compute(buf);
        __builtin_amdgcn_sched_barrier(0);
        lstore(ra0, rw0, buf ^ 1);
        __syncthreads();
      }
    }

    // ---- epilogue: lane owns columns 4*(lane/16)+0..3 of token row lane%16 ----
    constexpr int FO = SWI ? FW / 2 : FW;
    const int wcol0 = SWI ? wn * (WTW / 2) : wn * WTW;
#pragma unroll
    for (int i = 0; i < FO; ++i) {
      const int col = n0 + wcol0 + i * 16 + 4 * lch;
      if (col >= a.n_out) continue;
      float bias[4] = {0.f, 0.f, 0.f, 0.f};
      if (MODE != kUpSwiglu && a.bias && g < a.E) {
        const uint2 b = *reinterpret_cast<const uint2 *>(a.bias + (int64_t)g * a.n_out + col);
        bias[0] = __uint_as_float(b.x << 16);
        bias[1] = __uint_as_float(b.x & 0xffff0000u);
        bias[2] = __uint_as_float(b.y << 16);
        bias[3] = __uint_as_float(b.y & 0xffff0000u);
      }
#pragma unroll
      for (int j = 0; j < FM; ++j) {
        const int m = m0 + wm * WTM + j * 16 + lrow;
        if (m >= rows) continue;
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if constexpr (MODE == kUpSwiglu) {
            v[r] = silu_f32(acc[i][j][r]) * acc[i + FW / 2][j][r];
          } else if constexpr (MODE == kUpGelu) {
            v[r] = gelu_f32(acc[i][j][r] + bias[r]);
          } else {
            v[r] = acc[i][j][r] + bias[r];
          }
        }
        uint2 o;
        o.x = pack_bf16x2(v[0], v[1]);
        o.y = pack_bf16x2(v[2], v[3]);
        *reinterpret_cast<uint2 *>(a.c + (int64_t)(grow0 + m) * a.n_out + col) = o;
      }
    }
  }
}

// ---------------------------------------------------------------- launch --

static int num_cus() {
  static int cached = 0;
  if (!cached) {
    int dev = 0;
    hipGetDevice(&dev);
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached = n;
  }
  return cached;
}

// persistent: one resident wave of workgroups walks all tiles; otherwise one
// workgroup per tile (the hardware dispatcher balances short streaming tiles)
template <int BM, int BNW, int WM, int WN, int BK, int PFD, int MODE, bool PERSIST = true>
static hipError_t launch_bm(const GemmArgs &a0, hipStream_t s) {
  constexpr int NT = WM * WN * 64;
  GemmArgs a = a0;
  constexpr int BN_OUT = MODE == kUpSwiglu ? BNW / 2 : BNW;
  a.n_tiles = (a.n_out + BN_OUT - 1) / BN_OUT;
  // upper bound of the ragged m-tile count: every group wastes < 1 tile
  const int64_t mt_bound = (int64_t)(a.routed_rows + BM - 1) / BM + a.E + a.S;
  const int64_t tiles = mt_bound * a.n_tiles;
  static int per_cu = 0;   // resident workgroups per CU for this instantiation
  if (!per_cu) {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &nb, gemm_bf16_kernel<BM, BNW, WM, WN, BK, PFD, MODE>, NT, 0) != hipSuccess || nb <= 0)
      nb = 1;
    per_cu = nb;
  }
  int64_t grid = (int64_t)num_cus() * per_cu;   // persistent grid
  if (!PERSIST || tiles < grid) grid = tiles;
  grid = ((grid + 7) / 8) * 8;     // the slice order needs a multiple of 8
  gemm_bf16_kernel<BM, BNW, WM, WN, BK, PFD, MODE><<<(int)grid, NT, 0, s>>>(a);
  return hipGetLastError();
}

// Groups are split by row count into two tile classes, one launch each:
// small groups (<= 64 rows: decode batches, cold experts) stream their
// weights through 32-row tiles; larger groups use 256 x 256 tiles.  The
// large class is skipped when no group can exceed 64 rows (every group has
// at most T rows).
template <int MODE>
static hipError_t launch_classes(GemmArgs a, hipStream_t s) {
  hipError_t err = hipSuccess;
  if (a.T > 64) {
    a.min_rows = 65;
    a.max_rows = 1 << 30;
    if ((err = launch_bm<256, 256, 4, 2, 64, 1, MODE>(a, s)) != hipSuccess) return err;
  }
  a.min_rows = 1;
  a.max_rows = 64;
  return launch_bm<32, 128, 2, 2, 64, 2, MODE>(a, s);
}

hipError_t launch_expert_up_bf16(bool swiglu, const int32_t *offsets, int E, int S,
                                 int T, int k, int d, int h, const void *x_perm,
                                 const void *x, const void *w_up,
                                 const void *w_up_shared, const void *b_up,
                                 void *hidden, hipStream_t s) {
  GemmArgs a{};
  a.offsets = offsets;
  a.E = E;
  a.S = S;
  a.T = T;
  a.routed_rows = T * k;
  a.a_routed = static_cast<const uint16_t *>(x_perm);
  a.a_shared = static_cast<const uint16_t *>(x);
  a.K = d;
  a.w = static_cast<const uint16_t *>(w_up);
  a.w_shared = static_cast<const uint16_t *>(w_up_shared);
  a.w_rows = swiglu ? 2 * h : h;
  a.bias = static_cast<const uint16_t *>(b_up);
  a.c = static_cast<uint16_t *>(hidden);
  a.n_out = h;
  return swiglu ? launch_classes<kUpSwiglu>(a, s) : launch_classes<kUpGelu>(a, s);
}

hipError_t launch_expert_down_bf16(const int32_t *offsets, int E, int S, int T,
                                   int k, int d, int h, const void *hidden,
                                   const void *w_down, const void *w_down_shared,
                                   const void *b_down, void *y_perm,
                                   hipStream_t s) {
  GemmArgs a{};
  a.offsets = offsets;
  a.E = E;
  a.S = S;
  a.T = T;
  a.routed_rows = T * k;
  a.a_routed = static_cast<const uint16_t *>(hidden);
  a.a_shared = static_cast<const uint16_t *>(hidden) + (int64_t)T * k * h;
  a.K = h;
  a.w = static_cast<const uint16_t *>(w_down);
  a.w_shared = static_cast<const uint16_t *>(w_down_shared);
  a.w_rows = d;
  a.bias = static_cast<const uint16_t *>(b_down);
  a.c = static_cast<uint16_t *>(y_perm);
  a.n_out = d;
  return launch_classes<kDown>(a, s);
}

}  // namespace moe
