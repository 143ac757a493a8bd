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
// Both operands are K-contiguous, so tiles of either are runs of rows along
// K.  The MFMA is v_mfma_f32_16x16x32_bf16 with the weight rows as its A
// operand (M side) and the token rows as its B operand (N side): a lane then
// owns 4 consecutive output columns of one token row, and the epilogue
// stores 8-byte runs.  fp32 accumulation in registers.
//
// A persistent grid walks the ragged tile space: every workgroup computes
// the per-group tile prefix from the group offsets (no host sync), then
// takes tiles in a slice order that keeps each XCD (workgroups are dealt to
// the 8 XCDs round-robin) on a contiguous run of tiles, i.e. the m-tiles of
// a few neighbouring weight tiles, so weight tiles are fetched from HBM once
// per XCD and reused from its L2.  Three kernels share the tile arithmetic:
//
//   gemm_dma_kernel   large groups (row-major weights: K <= 8192): operands
//                     DMA'd from global memory into four rotating LDS
//                     buffers, 8 waves
//   gemm_pp_kernel    large groups, row-major weights, longer K: register-
//                     staged loads, two wave groups alternating compute and
//                     memory slots
//   gemm_bf16_kernel  small groups (<= 64 rows, e.g. decode): 32- or 64-row tiles
//                     streaming the weights, registers -> LDS, lock-step
//
// Measured on MI355X the large-group kernels are bound by the L2 -> CU
// operand stream (about 21-26 B/clk per CU over row-major weights, against
// 32 B/clk that full MFMA rate on 256 x 256 tiles would need), not by LDS.
// The texture path's cost goes by the cache lines a load touches: a 16-row
// x 64-byte block is 16 half lines, so weights in the tiled order (each
// such block stored as 1 KB of contiguous memory) load at twice the bytes
// per cycle; the token rows, gathered from any row, stay row-major.
#include "common.h"

#include <algorithm>
#include <cmath>

namespace moe {

// Up modes with Pre also store the pre-activations (SwiGLU: gate and up
// rows; GELU: x W1^T + b1) for the backward pass of a training step.
// kDownKN: the plain map of kDown with each group's weight matrix stored
// [K][N] (N contiguous), as the backward pass finds W2 and W1 for dH = dY W2
// and dX = dA W1; its MFMA fragments come from LDS through transposing
// reads.
enum GemmMode { kUpGelu = 0, kUpSwiglu = 1, kDown = 2, kUpGeluPre = 3, kUpSwigluPre = 4,
                kDownKN = 5 };
constexpr bool mode_swiglu(int m) { return m == kUpSwiglu || m == kUpSwigluPre; }
constexpr bool mode_kn(int m) { return m == kDownKN; }
constexpr bool mode_gelu(int m) { return m == kUpGelu || m == kUpGeluPre; }
constexpr bool mode_pre(int m) { return m == kUpGeluPre || m == kUpSwigluPre; }

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
  uint16_t *c_pre;          // Pre modes: [routed_rows + S*T, w_rows] pre-activations
  // Gathered token rows (up projection): when set, grouped row p of a routed
  // group is row gather[p] of gather_x [T, K] (the dispatch's perm_src), so
  // the grouped copy x_perm is never written; a_routed is then unused
  const int32_t *gather;
  const uint16_t *gather_x;
  // Weights (w, w_shared) in the tiled layout: each [w_rows, K] matrix is a
  // grid of 1 KB blocks of 16 rows x 32 k, block (rb, kb) at byte
  // (rb * K/32 + kb) * 1024, 16-byte piece p of a block holding row p / 4 and
  // chunk (p % 4) ^ (p / 16) of the block (tile_weights_kernel writes it).
  // The launch picks the kernels compiled for that order (template flag WT).
  int w_tiled;
};

// Weight-load addressing of the register-staged kernels: load i of stage kt
// reads byte v0 + i * istride + kt * kstep of the tile's weight descriptor.
struct WAddr {
  uint32_t v0, istride;
  int kstep;
};

// Word 3 of a raw buffer resource on gfx9-family parts (32-bit data format,
// no swizzle, no index stride).
constexpr int kBufferWord3 = 0x00020000;

// LDS placement of 16-byte chunk `chunk` of tile row `row`.  With 32-wide
// k stages a row is 64 B and 16 rows fill one 1 KB block; in a fragment read
// 16 lanes read one chunk of 16 consecutive rows, which unswizzled fall on
// only 4 distinct 16-byte slots of the 256-byte bank row.  XOR-ing the chunk
// with bits 2-3 of the row spreads the 16 rows over 16 slots.  (Measured on
// MI355X the k32 DMA kernel's bank-conflict counter is the same with and
// without this swizzle, and so is its time: its conflicts come from another
// access.)  With 64-wide stages the 128-B rows are XOR-swizzled (pattern
// chosen by measuring fragment-read throughput and whole-kernel time against
// a k32-plane layout).  The swizzle is an XOR, so it is its own inverse:
// swz(swz(c, r), r) = c.
template <int BK>
__device__ __forceinline__ int swz(int chunk, int row) {
  if constexpr (BK == 32) return chunk ^ ((row >> 2) & 3);
  return chunk ^ ((((row >> 2) & 3) << 1) ^ ((row >> 1) & 1));
}

// DMA lane map of a k32 stage: lane l of a 16-row block (first row a
// multiple of 16) fills LDS slot l, i.e. row l / 4, physical chunk l % 4,
// which holds logical chunk swz(l % 4, l / 4) = (l % 4) ^ (l / 16).
__device__ __forceinline__ uint32_t dma32_chunk_bytes(int lane) {
  return (uint32_t)swz<32>(lane % 4, lane / 4) * 16u;
}

// Workgroup barrier that orders LDS only: the wave waits for its own LDS
// operations, not for its global loads, which stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Per-group m-tile prefix (exclusive) of the groups this launch takes, into
// tprefix[0..G]; robust against out-of-range offsets.  Thread t owns groups
// 2t and 2t+1 (G <= 257 <= 2 * NT).
template <int NT, int BM>
__device__ __forceinline__ void tile_prefix(const GemmArgs &a, int *tprefix, int *scan_tmp) {
  static_assert(2 * NT >= kMaxExperts + 1, "two groups per thread cover E + S");
  const int tid = threadIdx.x;
  const int G = a.E + a.S;
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

// One output tile: group, row range and the buffer descriptors of its
// operands.  Loads past the last valid row (group tail, N tail) are out of
// the descriptor's range and return zeros, so no clamping is needed and one
// 32-bit offset per thread addresses all of its 16-byte loads.
struct Tile {
  int g, grow0, rows, m0, n0;
  int hv;              // token rows of the tile that it computes and stores
  bool gather;         // token rows gathered from GemmArgs::gather_x
  __amdgpu_buffer_rsrc_t rs_a, rs_w0, rs_w1;
  uint32_t w_stride;   // kDownKN: bytes per k row of the weights
};

// Byte offset (from the tile's A descriptor) of the start of tile-local
// token row r.  Gathered rows: row gather[p] of x, the descriptor covering
// all of x; a row past the tile's rows (t.hv) gets offset T * row_bytes, out
// of the descriptor's range, so it reads zeros (as does a corrupt index).
// Otherwise the descriptor starts at the tile's first row and ends with its
// last one.
__device__ __forceinline__ uint32_t a_row_offset(const GemmArgs &a, const Tile &t, int r,
                                                 uint32_t row_bytes) {
  if (t.gather) {
    int src = a.T;
    if (r < t.hv) {
      const int p = a.gather[t.grow0 + t.m0 + r];
      if ((unsigned)p < (unsigned)a.T) src = p;
    }
    return (uint32_t)src * row_bytes;
  }
  return (uint32_t)r * row_bytes;
}

// Tile L of the launch's ragged tile space: group g owns tiles
// [tprefix[g] * n_tiles, tprefix[g+1] * n_tiles), m-tile fastest.  A group
// of `rows` rows has mt = ceil(rows / BM) m-tiles, and they split its rows
// evenly: each takes hb = rows / mt rounded up to 16 rows (hb <= BM), the
// last one the rest.  A group of 1100 rows thus runs as 5 tiles of 224 rows
// rather than 4 full tiles and one of 76 rows padded to BM, and the rows
// past hb in a tile are neither read nor computed (the large-group kernel
// skips their MFMAs), so the padded work shrinks from up to BM - 1 rows per
// group to under 16 rows per tile.
template <int BM, int BNW, bool SWI, bool KN = false>
__device__ __forceinline__ Tile decode_tile(const GemmArgs &a, const int *tprefix, int L) {
  const int G = a.E + a.S;
  int lo = 0, hi = G - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) / 2;
    if (tprefix[mid] * a.n_tiles <= L) lo = mid; else hi = mid - 1;
  }
  // tile coordinates are workgroup-uniform: make that explicit so group
  // bases and buffer descriptors live in scalar registers
  Tile t;
  t.g = __builtin_amdgcn_readfirstlane(lo);
  const int tpg = __builtin_amdgcn_readfirstlane(tprefix[t.g]);
  const int tg = __builtin_amdgcn_readfirstlane(tprefix[t.g + 1]) - tpg;
  const int local = L - tpg * a.n_tiles;
  const int nt = local / tg;
  const int mt = local % tg;
  const uint16_t *abase;
  const uint16_t *wbase;
  if (t.g < a.E) {
    const int r0 = min(max(a.offsets[t.g], 0), a.routed_rows);
    const int r1 = min(max(a.offsets[t.g + 1], r0), a.routed_rows);
    t.grow0 = r0;
    t.rows = r1 - r0;
    abase = a.a_routed + (int64_t)r0 * a.K;   // (unused for gathered rows)
    wbase = a.w + (int64_t)t.g * a.w_rows * a.K;
  } else {
    t.grow0 = a.routed_rows;
    t.rows = a.T;
    abase = a.a_shared;
    wbase = a.w_shared;
  }
  const int hb = min(BM, ((t.rows + tg - 1) / tg + 15) & ~15);
  t.m0 = mt * hb;
  t.hv = min(hb, t.rows - t.m0);
  t.n0 = nt * (SWI ? BNW / 2 : BNW);
  const uint32_t row_bytes = (uint32_t)a.K * 2u;
  const int arows = t.hv;
  t.gather = a.gather != nullptr && t.g < a.E;
  if (t.gather)
    t.rs_a = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(a.gather_x), 0,
                                               (uint32_t)a.T * row_bytes, kBufferWord3);
  else
    t.rs_a = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(abase + (int64_t)t.m0 * a.K), 0, arows * row_bytes, kBufferWord3);
  if constexpr (KN) {
    // [K][w_rows] weights: columns n0.. of every k row; the range ends with
    // the group's matrix, so stages past K read zeros
    t.w_stride = (uint32_t)a.w_rows * 2u;
    t.rs_w0 = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(wbase + t.n0), 0,
        (uint32_t)(((int64_t)a.K * a.w_rows - t.n0) * 2), kBufferWord3);
    t.rs_w1 = t.rs_w0;
  } else if constexpr (SWI) {
    const int h = a.n_out;
    const int wv = min(BNW / 2, h - t.n0);
    t.rs_w0 = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(wbase + (int64_t)t.n0 * a.K), 0, wv * row_bytes, kBufferWord3);
    t.rs_w1 = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(wbase + (int64_t)(h + t.n0) * a.K), 0, wv * row_bytes, kBufferWord3);
  } else {
    const int wv = min(BNW, a.w_rows - t.n0);
    t.rs_w0 = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(wbase + (int64_t)t.n0 * a.K), 0, wv * row_bytes, kBufferWord3);
    t.rs_w1 = t.rs_w0;
  }
  return t;
}

// Tile arithmetic shared by the kernels: BM token rows x BNW weight rows per
// tile, k stages of BK, WM x WN waves each owning (BM/WM) x (BNW/WN).
// LDS layout of a stage: XOR-swizzled 128-byte rows, or (PLANES) BK/32
// planes of 64-byte rows, where every 16-row fragment read and every
// 16-row x 64-byte store is one contiguous 1 KB block.
template <int BM, int BNW, int WM, int WN, int BK, int MODE, bool PLANES = false>
struct TileMath {
  static constexpr int NT = WM * WN * 64;
  static constexpr int CH = BK / 8;            // 16-byte chunks per row
  static constexpr int KS = BK / 32;           // k32 MFMA steps per stage
  static constexpr int WTM = BM / WM;          // token rows per wave
  static constexpr int WTW = BNW / WN;         // weight rows per wave
  static constexpr int FM = WTM / 16;
  static constexpr int FW = WTW / 16;
  static constexpr bool SWI = mode_swiglu(MODE);
  static constexpr int BN_OUT = SWI ? BNW / 2 : BNW;
  // kDownKN: a weight stage is BK rows of k, each BNW values of n (WCH
  // 16-byte chunks); chunk c of row k sits at c ^ (k & 7), so the four k
  // rows a transposing read touches fall in different banks
  static constexpr bool KN = mode_kn(MODE);
  static constexpr int WCH = BNW / 8;
  static_assert(!KN || (WCH >= 8 && !PLANES), "k-row weight stage");
  static __device__ __forceinline__ int kn_slot(int k, int c) { return k * WCH + (c ^ (k & 7)); }
  // Token rows of fragment j of wave row wm: the waves' fragments
  // interleave (fragment j of the WM wave rows covers rows 16 (j WM + wm)
  // .. + 15), so that when a tile computes only its first hv rows every
  // wave row drops the same number of fragments, give or take one, and the
  // SIMDs (two wave rows each) stay evenly loaded.
  static __device__ __forceinline__ int frag_row(int wm, int j) { return (j * WM + wm) * 16; }
  static constexpr int A_LD = BM * CH / NT;    // 16-byte loads per thread per stage
  static constexpr int W_LD = BNW * CH / NT;
  static_assert(BK == 32 || BK == 64, "stage depth");
  static_assert(FM >= 1 && FW >= 1 && (!SWI || FW % 2 == 0), "wave tile");

  // thread's first row (tid / CH) and 16-byte chunk (tid % CH); load i
  // covers row tid / CH + i * (NT / CH)
  static __device__ __forceinline__ uint32_t voff0(uint32_t row_bytes) {
    return (uint32_t)(threadIdx.x / CH) * row_bytes + (uint32_t)(threadIdx.x % CH) * 16u;
  }
  // per-thread offsets of the A loads of tile t (gathered or contiguous rows)
  static __device__ __forceinline__ void a_offsets(const GemmArgs &a, const Tile &t,
                                                   uint32_t row_bytes, uint32_t (&va)[A_LD]) {
#pragma unroll
    for (int i = 0; i < A_LD; ++i)
      va[i] = a_row_offset(a, t, (int)(threadIdx.x / CH) + i * (NT / CH), row_bytes) +
              (uint32_t)(threadIdx.x % CH) * 16u;
  }

  // The thread's weight loads: row tid / CH + i * (NT / CH), chunk tid % CH
  // as for the token rows.  Row-major weights: from the tile's first row;
  // tiled weights: the same row and chunk inside its 16 x 32 block, so that
  // a wavefront's loads cover whole 1 KB blocks (whole 128-byte lines).
  template <bool WT>
  static __device__ __forceinline__ WAddr waddr(const GemmArgs &a, uint32_t row_bytes) {
    WAddr w;
    if constexpr (WT) {
      static_assert((NT / CH) % 16 == 0, "a load's rows span whole blocks");
      const uint32_t nkb = (uint32_t)a.K / 32u;
      const int r = threadIdx.x / CH, c = threadIdx.x % CH;
      const int rr = r % 16;
      w.v0 = ((uint32_t)(r / 16) * nkb + (uint32_t)(c / 4)) * 1024u +
             (uint32_t)(rr * 4 + ((c % 4) ^ (rr / 4))) * 16u;
      w.istride = (uint32_t)(NT / CH / 16) * nkb * 1024u;
      w.kstep = (BK / 32) * 1024;
    } else {
      w.v0 = voff0(row_bytes);
      w.istride = (uint32_t)(NT / CH) * row_bytes;
      w.kstep = BK * 2;
    }
    return w;
  }

  // register-staged stage loads: every thread moves A_LD + W_LD chunks
  static constexpr void check_load_split() {
    static_assert(A_LD * NT == BM * CH && W_LD * NT == BNW * CH, "load split");
    static_assert(!SWI || (W_LD % 2 == 0), "gate and up rows split the loads evenly");
  }
  static __device__ __forceinline__ void gload(const Tile &t, const WAddr &wa,
                                               const uint32_t (&va)[A_LD],
                                               u32x4_t (&ra)[A_LD], u32x4_t (&rw)[W_LD], int kt) {
    check_load_split();
    // the k offset is uniform: it goes in the scalar offset, so the vector
    // offsets stay loop-invariant (row validity is decided by them alone)
    const int ko = kt * (BK * 2);
#pragma unroll
    for (int i = 0; i < A_LD; ++i)
      ra[i] = __builtin_amdgcn_raw_buffer_load_b128(t.rs_a, va[i], ko, 0);
    if constexpr (KN) {
      // chunk q: k row q / WCH of the stage, 16-byte chunk q % WCH
#pragma unroll
      for (int i = 0; i < W_LD; ++i) {
        const int q = (int)threadIdx.x + i * NT;
        rw[i] = __builtin_amdgcn_raw_buffer_load_b128(
            t.rs_w0, (uint32_t)(q / WCH) * t.w_stride + (uint32_t)(q % WCH) * 16u,
            (int)((uint32_t)(kt * BK) * t.w_stride), 0);
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < W_LD; ++i) {
      if (!SWI || i < W_LD / 2) {
        rw[i] = __builtin_amdgcn_raw_buffer_load_b128(t.rs_w0, wa.v0 + i * wa.istride,
                                                      kt * wa.kstep, 0);
      } else {
        rw[i] = __builtin_amdgcn_raw_buffer_load_b128(
            t.rs_w1, wa.v0 + (i - W_LD / 2) * wa.istride, kt * wa.kstep, 0);
      }
    }
  }

  static __device__ __forceinline__ void lstore(u32x4_t *As, u32x4_t *Ws,
                                                const u32x4_t (&ra)[A_LD],
                                                const u32x4_t (&rw)[W_LD]) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < A_LD; ++i) {
      const int q = tid + i * NT;
      As[(q / CH) * CH + swz<BK>(q % CH, q / CH)] = ra[i];
    }
#pragma unroll
    for (int i = 0; i < W_LD; ++i) {
      const int q = tid + i * NT;
      if constexpr (KN)
        Ws[kn_slot(q / WCH, q % WCH)] = rw[i];
      else
        Ws[(q / CH) * CH + swz<BK>(q % CH, q / CH)] = rw[i];
    }
  }

  // LDS row of weight fragment i of wave column wn (SwiGLU: gate fragments
  // first, then the matching up fragments from the second half of the tile)
  static __device__ __forceinline__ int wrow(int wn, int i, int lrow) {
    if constexpr (SWI) {
      return (i < FW / 2) ? wn * (WTW / 2) + i * 16 + lrow
                          : BNW / 2 + wn * (WTW / 2) + (i - FW / 2) * 16 + lrow;
    } else {
      return wn * WTW + i * 16 + lrow;
    }
  }

  static constexpr int NWF = KS * FW;   // weight fragments per stage
  // weight fragments read ahead of the MFMAs that use them
  static constexpr int PD = (8 + FM - 1) / FM < NWF ? (8 + FM - 1) / FM : NWF;

  // MFMA operands of one stage: token fragment (k32 step s, row block j)
  // and weight fragment n = s * FW + i
  struct Frags {
    bf16x8_t a[KS][FM];
    bf16x8_t w[NWF];
  };

  // LDS slot (16-byte units) of chunk ch of row r of the token / weight tile
  static __device__ __forceinline__ int a_idx(int r, int ch) {
    if constexpr (PLANES) return ((ch >> 2) * BM + r) * 4 + (ch & 3);
    return r * CH + swz<BK>(ch, r);
  }
  static __device__ __forceinline__ int w_idx(int r, int ch) {
    if constexpr (PLANES) return ((ch >> 2) * BNW + r) * 4 + (ch & 3);
    return r * CH + swz<BK>(ch, r);
  }

  static __device__ __forceinline__ bf16x8_t read_a(const u32x4_t *As, int s, int j, int wm) {
    const int lane = threadIdx.x % 64;
    const int ch = 4 * s + lane / 16;
    const int r = frag_row(wm, j) + lane % 16;
    return __builtin_bit_cast(bf16x8_t, As[a_idx(r, ch)]);
  }
  static __device__ __forceinline__ bf16x8_t read_w(const u32x4_t *Ws, int n, int wn) {
    const int lane = threadIdx.x % 64;
    if constexpr (KN) {
      // Two transposing reads (ds_read_b64_tr_b16).  In each 16-lane group
      // the result lane i, element j is element i % 4 of the 4-value row
      // whose address lane i / 4 + 4 j gave.  Lane 4 j + a of group g gives
      // k row 8 g + 4 h + j (read h = 0, 1), n values nb + 4 a .. + 3; lane
      // i then holds W[k0 + 8 g .. + 7][nb + i]: the fragment of n row i.
      typedef short v4s __attribute__((ext_vector_type(4)));
      const int g = lane / 16, sl = lane % 16;
      const int nn = wrow(wn, n % FW, 0) + 4 * (sl & 3);
      const int k0 = 32 * (n / FW) + 8 * g + (sl >> 2);
      const char *base = reinterpret_cast<const char *>(Ws);
      const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) v4s *)(base + kn_slot(k0, nn >> 3) * 16 +
                                                    (nn & 7) * 2));
      const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) v4s *)(base + kn_slot(k0 + 4, nn >> 3) * 16 +
                                                    (nn & 7) * 2));
      typedef short v8s __attribute__((ext_vector_type(8)));
      const v8s both = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      return __builtin_bit_cast(bf16x8_t, both);
    }
    const int ch = 4 * (n / FW) + lane / 16;
    const int r = wrow(wn, n % FW, lane % 16);
    return __builtin_bit_cast(bf16x8_t, Ws[w_idx(r, ch)]);
  }

  // Token fragments of every k32 step and the first PD weight fragments.
  static __device__ __forceinline__ void head(const u32x4_t *As, const u32x4_t *Ws, Frags &f,
                                              int wm, int wn) {
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int j = 0; j < FM; ++j) f.a[s][j] = read_a(As, s, j, wm);
#pragma unroll
    for (int n = 0; n < PD; ++n) f.w[n] = read_w(Ws, n, wn);
  }

  // The stage's MFMAs; the remaining weight fragments are streamed PD ahead
  // of their first use.  LEAD: the head's reads are in the same scheduling
  // region and go first.
  template <bool LEAD>
  static __device__ __forceinline__ void body(const u32x4_t *Ws, Frags &f,
                                              f32x4_t (&acc)[FW][FM], int wn) {
#pragma unroll
    for (int n = PD; n < NWF; ++n) f.w[n] = read_w(Ws, n, wn);
#pragma unroll
    for (int n = 0; n < NWF; ++n)
#pragma unroll
      for (int j = 0; j < FM; ++j)
        acc[n % FW][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.w[n], f.a[n / FW][j],
                                                                 acc[n % FW][j], 0, 0, 0);
    if constexpr (LEAD) __builtin_amdgcn_sched_group_barrier(0x100, KS * FM + PD, 0);
#pragma unroll
    for (int n = 0; n < NWF; ++n) {
      __builtin_amdgcn_sched_group_barrier(0x008, FM, 0);
      if (n + PD < NWF) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
  }

  // One whole stage: head and body in one scheduling region.
  static __device__ __forceinline__ void compute(const u32x4_t *As, const u32x4_t *Ws,
                                                 f32x4_t (&acc)[FW][FM], int wm, int wn) {
    Frags f;
    head(As, Ws, f, wm, wn);
    body<true>(Ws, f, acc, wn);
  }

  // lane owns columns 4*(lane/16)+0..3 of token row lane%16 of each fragment;
  // values are computed unconditionally and only the stores are predicated,
  // which keeps the epilogue one basic block
  static __device__ __forceinline__ void epilogue(const GemmArgs &a, const Tile &t,
                                                  const f32x4_t (&acc)[FW][FM], int wm, int wn) {
    const int lane = threadIdx.x % 64;
    const int lrow = lane % 16;
    const int lch = lane / 16;
    constexpr int FO = SWI ? FW / 2 : FW;
    const int wcol0 = SWI ? wn * (WTW / 2) : wn * WTW;
    const bool has_bias = !mode_swiglu(MODE) && a.bias && t.g < a.E;
#pragma unroll
    for (int i = 0; i < FO; ++i) {
      const int col = t.n0 + wcol0 + i * 16 + 4 * lch;
      const bool col_ok = col < a.n_out;
      float bias[4] = {0.f, 0.f, 0.f, 0.f};
      if (has_bias && col_ok) {
        const uint2 b = *reinterpret_cast<const uint2 *>(a.bias + (int64_t)t.g * a.n_out + col);
        bias[0] = __uint_as_float(b.x << 16);
        bias[1] = __uint_as_float(b.x & 0xffff0000u);
        bias[2] = __uint_as_float(b.y << 16);
        bias[3] = __uint_as_float(b.y & 0xffff0000u);
      }
#pragma unroll
      for (int j = 0; j < FM; ++j) {
        const int lr = frag_row(wm, j) + lrow;   // tile-local row
        const int m = t.grow0 + t.m0 + lr;
        const bool row_ok = lr < t.hv;
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if constexpr (mode_swiglu(MODE)) {
            v[r] = silu_f32(acc[i][j][r]) * acc[i + FW / 2][j][r];
          } else if constexpr (mode_gelu(MODE)) {
            v[r] = gelu_f32(acc[i][j][r] + bias[r]);
          } else {
            v[r] = acc[i][j][r] + bias[r];
          }
        }
        uint2 o;
        o.x = pack_bf16x2(v[0], v[1]);
        o.y = pack_bf16x2(v[2], v[3]);
        if (col_ok && row_ok)
          *reinterpret_cast<uint2 *>(a.c + (int64_t)m * a.n_out + col) = o;
        if constexpr (mode_pre(MODE)) {
          // pre-activations: row stride w_rows (2h SwiGLU, h GELU)
          uint16_t *pre = a.c_pre + (int64_t)m * a.w_rows + col;
          uint2 p;
          if constexpr (mode_swiglu(MODE)) {
            p.x = pack_bf16x2(acc[i][j][0], acc[i][j][1]);
            p.y = pack_bf16x2(acc[i][j][2], acc[i][j][3]);
            uint2 u;
            u.x = pack_bf16x2(acc[i + FW / 2][j][0], acc[i + FW / 2][j][1]);
            u.y = pack_bf16x2(acc[i + FW / 2][j][2], acc[i + FW / 2][j][3]);
            if (col_ok && row_ok) {
              *reinterpret_cast<uint2 *>(pre) = p;
              *reinterpret_cast<uint2 *>(pre + a.n_out) = u;
            }
          } else {
            p.x = pack_bf16x2(acc[i][j][0] + bias[0], acc[i][j][1] + bias[1]);
            p.y = pack_bf16x2(acc[i][j][2] + bias[2], acc[i][j][3] + bias[3]);
            if (col_ok && row_ok) *reinterpret_cast<uint2 *>(pre) = p;
          }
        }
        // one output fragment at a time: keeps the scheduler from pulling
        // every accumulator into VGPRs at once
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  // The same outputs through LDS (not for the Pre modes): each lane puts
  // its 4 columns of a fragment row into a staging tile of BM rows x BN_OUT
  // bf16 (16-byte chunks XOR-swizzled by row, so that the 16 rows a fragment
  // writes and the chunks a row read takes fall in distinct banks), then
  // every thread stores whole 16-byte chunks of output rows: a store
  // instruction covers 4 rows x 256 contiguous bytes instead of 16 rows x
  // 32 bytes.  stage: BM * BN_OUT * 2 bytes of LDS that no wave still
  // reads; the caller puts a barrier after the call before reusing it.
  // n_out is a multiple of 64, so no chunk straddles the matrix edge.
  static __device__ __forceinline__ void epilogue_staged(const GemmArgs &a, const Tile &t,
                                                         const f32x4_t (&acc)[FW][FM], int wm,
                                                         int wn, u32x4_t *stage) {
    static_assert(!mode_pre(MODE), "pre-activations take the direct epilogue");
    constexpr int NCH = BN_OUT / 8;   // 16-byte chunks per staged row
    static_assert(NCH % 16 == 0, "row swizzle over 16 chunks");
    const int lane = threadIdx.x % 64;
    const int lrow = lane % 16;
    const int lch = lane / 16;
    constexpr int FO = SWI ? FW / 2 : FW;
    const int wcol0 = SWI ? wn * (WTW / 2) : wn * WTW;
    const bool has_bias = !mode_swiglu(MODE) && a.bias && t.g < a.E;
    char *sb = reinterpret_cast<char *>(stage);
#pragma unroll
    for (int i = 0; i < FO; ++i) {
      const int lc = wcol0 + i * 16 + 4 * lch;   // tile-local column
      const int col = t.n0 + lc;
      float bias[4] = {0.f, 0.f, 0.f, 0.f};
      if (has_bias && col < a.n_out) {
        const uint2 b = *reinterpret_cast<const uint2 *>(a.bias + (int64_t)t.g * a.n_out + col);
        bias[0] = __uint_as_float(b.x << 16);
        bias[1] = __uint_as_float(b.x & 0xffff0000u);
        bias[2] = __uint_as_float(b.y << 16);
        bias[3] = __uint_as_float(b.y & 0xffff0000u);
      }
#pragma unroll
      for (int j = 0; j < FM; ++j) {
        const int r = frag_row(wm, j) + lrow;   // tile-local row
        float v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if constexpr (mode_swiglu(MODE)) {
            v[q] = silu_f32(acc[i][j][q]) * acc[i + FW / 2][j][q];
          } else if constexpr (mode_gelu(MODE)) {
            v[q] = gelu_f32(acc[i][j][q] + bias[q]);
          } else {
            v[q] = acc[i][j][q] + bias[q];
          }
        }
        uint2 o;
        o.x = pack_bf16x2(v[0], v[1]);
        o.y = pack_bf16x2(v[2], v[3]);
        *reinterpret_cast<uint2 *>(sb + r * (NCH * 16) + (((lc >> 3) ^ (r & 15)) << 4) +
                                   (lc & 4) * 2) = o;
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __syncthreads();
    const int rows_valid = t.hv;
    const int cols_valid = min(BN_OUT, a.n_out - t.n0);
    for (int c = threadIdx.x; c < BM * NCH; c += NT) {
      const int r = c / NCH, q = c % NCH;
      if (r < rows_valid && q * 8 < cols_valid)
        *reinterpret_cast<u32x4_t *>(a.c + (int64_t)(t.grow0 + t.m0 + r) * a.n_out + t.n0 +
                                     q * 8) = stage[r * NCH + (q ^ (r & 15))];
    }
  }
};

// slice order: XCD x (= blockIdx % 8, workgroups are dealt to the XCDs
// round-robin) takes a contiguous run of tiles
__device__ __forceinline__ int slice_tile(int it) {
  const int nblk = gridDim.x;
  return it * nblk + (blockIdx.x % 8) * (nblk / 8) + blockIdx.x / 8;
}

// Lock-step kernel: every wave loads, stores and computes each stage; the
// loads of stage k+1 (PFD 1) or k+2 (PFD 2, register double buffer) fly
// while stage k is computed.  At least two waves per SIMD: 8-wave tiles run
// one workgroup per CU, 4-wave tiles two (their register budget is capped
// at 256 per lane).
template <int BM, int BNW, int WM, int WN, int BK, int PFD, int MODE, bool WT>
__global__ __launch_bounds__(WM *WN * 64) __attribute__((amdgpu_waves_per_eu(2)))
void gemm_bf16_kernel(GemmArgs a) {
  using TM = TileMath<BM, BNW, WM, WN, BK, MODE>;
  constexpr int NT = TM::NT, CH = TM::CH, A_LD = TM::A_LD, W_LD = TM::W_LD;
  constexpr int FM = TM::FM, FW = TM::FW;

  __shared__ u32x4_t As[2][BM * CH];
  __shared__ u32x4_t Ws[2][BNW * CH];
  __shared__ int tprefix[2 * NT + 2];
  __shared__ int scan_tmp[NT / 64];

  const int wave = threadIdx.x / 64;
  const int wm = wave / WN;
  const int wn = wave % WN;
  tile_prefix<NT, BM>(a, tprefix, scan_tmp);
  __syncthreads();
  const int total_tiles = tprefix[a.E + a.S] * a.n_tiles;
  const int nk = a.K / BK;
  const uint32_t row_bytes = (uint32_t)a.K * 2u;
  const WAddr wa = TM::template waddr<WT>(a, row_bytes);

  for (int it = 0;; ++it) {
    const int L = slice_tile(it);
    if (L >= total_tiles) break;
    const Tile t = decode_tile<BM, BNW, TM::SWI, TM::KN>(a, tprefix, L);
    uint32_t va[A_LD];
    TM::a_offsets(a, t, row_bytes, va);

    f32x4_t acc[FW][FM];
#pragma unroll
    for (int i = 0; i < FW; ++i)
#pragma unroll
      for (int j = 0; j < FM; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    u32x4_t ra0[A_LD], rw0[W_LD];
    u32x4_t ra1[PFD == 2 ? A_LD : 1], rw1[PFD == 2 ? W_LD : 1];

    // Scheduling fences keep each stage's global loads ahead of the MFMAs
    // (the compiler would otherwise sink them next to their LDS stores and
    // expose the whole load latency).
    if constexpr (PFD == 2) {
      TM::gload(t, wa, va, ra0, rw0, 0);
      TM::lstore(As[0], Ws[0], ra0, rw0);
      TM::gload(t, wa, va, ra1, rw1, 1);
      __syncthreads();
      int kt = 0;
      for (; kt + 2 <= nk; kt += 2) {
        // even step: LDS buffer 0 holds stage kt, registers 1 hold stage kt+1
        TM::gload(t, wa, va, ra0, rw0, kt + 2);
        __builtin_amdgcn_sched_barrier(0);
        TM::compute(As[0], Ws[0], acc, wm, wn);
        __builtin_amdgcn_sched_barrier(0);
        TM::lstore(As[1], Ws[1], ra1, rw1);
        __syncthreads();
        // odd step: LDS buffer 1 holds stage kt+1, registers 0 hold stage kt+2
        TM::gload(t, wa, va, ra1, rw1, kt + 3);
        __builtin_amdgcn_sched_barrier(0);
        TM::compute(As[1], Ws[1], acc, wm, wn);
        __builtin_amdgcn_sched_barrier(0);
        TM::lstore(As[0], Ws[0], ra0, rw0);
        __syncthreads();
      }
      if (kt < nk) TM::compute(As[0], Ws[0], acc, wm, wn);   // odd stage count
    } else {
      TM::gload(t, wa, va, ra0, rw0, 0);
      TM::lstore(As[0], Ws[0], ra0, rw0);
      __syncthreads();
      for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        TM::gload(t, wa, va, ra0, rw0, kt + 1);
        __builtin_amdgcn_sched_barrier(0);
        TM::compute(As[buf], Ws[buf], acc, wm, wn);
        __builtin_amdgcn_sched_barrier(0);
        TM::lstore(As[buf ^ 1], Ws[buf ^ 1], ra0, rw0);
        __syncthreads();
      }
    }
    TM::epilogue(a, t, acc, wm, wn);
  }
}

// Ping-pong kernel for large groups: BM x 256 tiles (BM = 256 or 192), 8
// waves in two groups of four, one wave of each group per SIMD.  The groups alternate between a
// compute slot (the MFMAs of one whole stage) and a memory slot (store the
// staged registers of the next stage to LDS, issue the global loads of the
// stage after it), offset by one slot, so that on every SIMD one wave feeds
// the matrix core while the other moves data.  Slots end at LDS-only
// barriers: global loads stay in flight for two slots.
//
// Group 0 (wave rows 0 and 1) computes stage k in slot 2k, group 1
// (the others) in slot 2k+1.  Group 1 stores its half of stage k+1 in slot
// 2k, group 0 in slot 2k+1, so stage k+1 is complete before slot 2k+2 and
// two LDS buffers suffice: stage k+2 overwrites stage k only from slot
// 2k+2 on, after both groups have finished it.
template <int BM, int MODE>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2)))
void gemm_pp_kernel(GemmArgs a) {
  constexpr int BNW = 256, WM = 4, WN = 2, BK = 64;
  using TM = TileMath<BM, BNW, WM, WN, BK, MODE>;
  constexpr int NT = TM::NT, CH = TM::CH, A_LD = TM::A_LD, W_LD = TM::W_LD;
  constexpr int FM = TM::FM, FW = TM::FW;

  // the two stage buffers (token, then weight); between tiles they also
  // stage the output tile
  __shared__ u32x4_t ring[2 * (BM + BNW) * CH];
  static_assert(BM * TM::BN_OUT * 2 <= 2 * (BM + BNW) * CH * 16, "output tile fits the ring");
  auto As = reinterpret_cast<u32x4_t(*)[BM * CH]>(ring);
  auto Ws = reinterpret_cast<u32x4_t(*)[BNW * CH]>(ring + 2 * BM * CH);
  __shared__ int tprefix[2 * NT + 2];
  __shared__ int scan_tmp[NT / 64];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
  const int wm = wave / WN;
  const int wn = wave % WN;
  const int grp = wave / 4;
  tile_prefix<NT, BM>(a, tprefix, scan_tmp);
  __syncthreads();
  const int total_tiles = tprefix[a.E + a.S] * a.n_tiles;
  const uint32_t row_bytes = (uint32_t)a.K * 2u;
  const WAddr wa = TM::template waddr<false>(a, row_bytes);
  const int nk = a.K / BK;

  for (int it = 0;; ++it) {
    const int L = slice_tile(it);
    if (L >= total_tiles) break;
    const Tile t = decode_tile<BM, BNW, TM::SWI, TM::KN>(a, tprefix, L);
    uint32_t va[A_LD];
    TM::a_offsets(a, t, row_bytes, va);

    f32x4_t acc[FW][FM];
#pragma unroll
    for (int i = 0; i < FW; ++i)
#pragma unroll
      for (int j = 0; j < FM; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    u32x4_t ra[A_LD], rw[W_LD];
    TM::gload(t, wa, va, ra, rw, 0);
    TM::lstore(As[0], Ws[0], ra, rw);
    if (nk > 1) TM::gload(t, wa, va, ra, rw, 1);
    __syncthreads();

    auto memory_slot = [&](int kt) {
      if (kt + 1 < nk) TM::lstore(As[(kt + 1) & 1], Ws[(kt + 1) & 1], ra, rw);
      if (kt + 2 < nk) TM::gload(t, wa, va, ra, rw, kt + 2);
    };
    // group 1 runs its memory slots one stage ahead; one call site each for
    // compute and memory keeps the register assignment identical for both
    // groups
    if (grp == 1) {
      memory_slot(0);
      lds_barrier();
    }
    for (int kt = 0; kt < nk; ++kt) {
      TM::compute(As[kt & 1], Ws[kt & 1], acc, wm, wn);
      lds_barrier();
      memory_slot(kt + grp);
      if (kt + grp < nk) lds_barrier();
    }
    // (every compute slot ended before the last barrier: the ring is free)
    if constexpr (mode_pre(MODE) || mode_gelu(MODE)) {
      TM::epilogue(a, t, acc, wm, wn);
    } else {
      TM::epilogue_staged(a, t, acc, wm, wn, ring);
      __syncthreads();   // the staged rows are read before the next stores
    }
  }
}

// A compile-time count, and the call f(IntC<c>) for c = clamp(n, 1, N)
// (a wave-uniform count picks one of N unrolled code paths).
template <int V>
struct IntC {
  static constexpr int value = V;
};
// f(IntC<c>) for c = clamp(n, 0, N)
template <int N, typename F>
__device__ __forceinline__ void with_count0(int n, F &&f) {
  if constexpr (N <= 0) {
    f(IntC<0>{});
  } else {
    if (n >= N) f(IntC<N>{});
    else with_count0<N - 1>(n, f);
  }
}
template <int N, typename F>
__device__ __forceinline__ void with_count(int n, F &&f) {
  if constexpr (N <= 1) {
    f(IntC<1>{});
  } else {
    if (n >= N) f(IntC<N>{});
    else with_count<N - 1>(n, f);
  }
}

// DMA-fed kernel for large groups: BM x BNW tiles (token rows x weight
// rows), WM x WN waves.  Operands go from global memory straight into LDS
// (buffer loads with the LDS flag): stores from registers would compete with
// the fragment reads for the LDS port, DMA writes barely do, and no staging
// registers are needed.  Stages are k32 wide (rows of 64 B, so a 16-row
// fragment read or a 16-row DMA block is one contiguous 1 KB) and rotate
// through four LDS buffers:
//
//   iteration s: read the operands of stage s+1 | MFMAs of stage s |
//                DMA stage s+4 (into the buffer of stage s, whose operands
//                are in registers by now) | wait for stage s+2 | barrier
//
// so the MFMAs after a barrier never wait for memory and a DMA has more
// than two iterations to land (L2 misses included).  DMAs and reads past
// the last stage stay in bounds (buffer descriptors; spare LDS buffers) and
// are never used; rows past the group's end or the weight matrix only feed
// outputs that the epilogue drops.
template <int BM, int BNW, int WM, int WN, int MODE, bool WT>
__global__ __launch_bounds__(WM *WN * 64) __attribute__((amdgpu_waves_per_eu(WM * WN / 4)))
void gemm_dma_kernel(GemmArgs a) {
  constexpr int BK = 32, NB = 4, NW = WM * WN;
  using TM = TileMath<BM, BNW, WM, WN, BK, MODE>;
  constexpr int NT = TM::NT, CH = TM::CH;
  constexpr int FM = TM::FM, FW = TM::FW;
  constexpr int ABLK = BM / 16, WBLK = BNW / 16;        // 16-row DMA blocks
  constexpr int NBLK = ABLK + WBLK;
  // blocks per wave.  A wave whose first block is past the stage's last
  // (the eighth wave of a 192-row tile: 28 blocks for 8 waves of 4) issues
  // no DMAs: its vmcnt wait is then empty, and the barrier after it still
  // waits for every other wave's.  Were a wave's blocks only partly past
  // the end, it would repeat the stage's last block (same data to the same
  // place), so that its vmcnt counts stages like everyone else's.
  constexpr int BPW = (NBLK + NW - 1) / NW;
  static_assert(CH == 4, "k32 stages");
  // interleave: QM MFMAs per operand read or DMA, then the rest
  constexpr int NMEM = FM + FW + BPW;
  constexpr int QM = (FW * FM) / NMEM >= 2 ? 2 : 1;
  static_assert(QM * NMEM <= FW * FM, "operand traffic fits the MFMA stream");

  // the operand ring (token buffers, then weight buffers); between tiles it
  // also stages the output tile
  __shared__ u32x4_t ring[NB * (BM + BNW) * CH];
  static_assert(BM * TM::BN_OUT * 2 <= NB * (BM + BNW) * CH * 16, "output tile fits the ring");
  auto As = reinterpret_cast<u32x4_t(*)[BM * CH]>(ring);
  auto Ws = reinterpret_cast<u32x4_t(*)[BNW * CH]>(ring + NB * BM * CH);
  __shared__ int tprefix[2 * NT + 2];
  __shared__ int scan_tmp[NT / 64];

  const int lane = threadIdx.x % 64;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
  const int wm = wave / WN;
  const int wn = wave % WN;
  tile_prefix<NT, BM>(a, tprefix, scan_tmp);
  __syncthreads();
  const int total_tiles = tprefix[a.E + a.S] * a.n_tiles;
  const uint32_t row_bytes = (uint32_t)a.K * 2u;
  // lane -> row lane / 4 of a 16-row block, the chunk its LDS slot holds;
  // tiled weights hold each 16-row block of a stage as 1 KB in LDS order
  const uint32_t voff = (uint32_t)(lane / 4) * row_bytes + dma32_chunk_bytes(lane);
  const int nk = a.K / BK;
  static_assert(!(WT && TM::KN), "k-row weights are row-major");

  for (int it = 0;; ++it) {
    const int L = slice_tile(it);
    if (L >= total_tiles) break;
    const Tile t = decode_tile<BM, BNW, TM::SWI, TM::KN>(a, tprefix, L);
    // offsets of this lane's token-row loads (row lane / 4 of each 16-row
    // token block the wave moves, gathered or contiguous); tiled weights:
    // the lane's 16 bytes of the weight block's first stage, so that the
    // scalar offset only steps through the stages
    uint32_t va[BPW];
#pragma unroll
    for (int i = 0; i < BPW; ++i) {
      const int blk = min(wave * BPW + i, NBLK - 1);   // wave-uniform
      if (blk < ABLK) {
        va[i] = a_row_offset(a, t, blk * 16 + lane / 4, row_bytes) + dma32_chunk_bytes(lane);
      } else if constexpr (WT) {
        const int wb = blk - ABLK;
        const int rb = TM::SWI && wb >= WBLK / 2 ? wb - WBLK / 2 : wb;   // block in its half
        va[i] = (uint32_t)(rb * nk) * 1024u + (uint32_t)lane * 16u;
      } else {
        va[i] = 0u;
      }
    }

    // wave w moves blocks BPW w .. BPW w + BPW - 1 of the stage: token
    // blocks first, then weight blocks (SwiGLU: gate rows from one
    // descriptor, up rows from the other).  It moves only the first ndma
    // of them: blocks past the stage's last one, and token blocks past the
    // tile's rows (no fragment of those rows is read), are left out.  They
    // are the last ones of the wave's run, since no run straddles the
    // token/weight boundary.  Each wave waits on its own count of DMAs (two
    // stages' worth stay in flight), and the stage barrier after the wait
    // covers the other waves' DMAs; the main loop is compiled for each
    // count, so the DMA issue and the waits stay branch-free.
    static_assert(ABLK % BPW == 0, "no wave moves both token and weight blocks");
    const int nvb = (t.hv + 15) / 16;
    int nd = min(BPW, max(0, NBLK - wave * BPW));
    if (wave * BPW < ABLK) nd = min(nd, max(0, nvb - wave * BPW));
    const int ndma = __builtin_amdgcn_readfirstlane(nd);
    // the wave's block i of stage s
    auto issue = [&](int i, int s) {
      const int blk = min(wave * BPW + i, NBLK - 1);
      __amdgpu_buffer_rsrc_t rs;
      u32x4_t *dst;
      int row = 0;
      if (blk < ABLK) {
        rs = t.rs_a;
        dst = As[s % NB] + blk * 64;
      } else {
        const int wb = blk - ABLK;
        dst = Ws[s % NB] + wb * 64;
        if constexpr (TM::KN) {
          // 64 / WCH k rows per block; lane -> physical chunk lane % WCH
          // of row kr, holding logical chunk (lane % WCH) ^ (kr & 7)
          constexpr int RPB = 64 / TM::WCH;
          const int kr = wb * RPB + lane / TM::WCH;
          const uint32_t vw = (uint32_t)(lane / TM::WCH) * t.w_stride +
                              (uint32_t)((lane % TM::WCH) ^ (kr & 7)) * 16u;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              t.rs_w0, dst, 16, vw, (int)((uint32_t)(s * BK + wb * RPB) * t.w_stride), 0, 0);
          return;
        }
        if (TM::SWI && wb >= WBLK / 2) {
          rs = t.rs_w1;
          row = (wb - WBLK / 2) * 16;
        } else {
          rs = t.rs_w0;
          row = wb * 16;
        }
      }
      // token blocks: the lane's own row offset (gathered rows); weight
      // blocks: the block's first row in the scalar offset (row-major), or
      // the block in the lane's offset and the stage's 1 KB step (tiled)
      const uint32_t vo = blk < ABLK || WT ? va[i] : voff;
      const int so = WT && blk >= ABLK ? s * 1024 : row * (int)row_bytes + s * (BK * 2);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 16, vo, so, 0, 0);
    };

    f32x4_t acc[FW][FM];
#pragma unroll
    for (int i = 0; i < FW; ++i)
#pragma unroll
      for (int j = 0; j < FM; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // The main loop for FV token fragments and ND DMAs per stage: fragments
    // FV.. of the wave cover rows past the tile's hv and are neither read
    // nor multiplied.  Every wave takes the same barriers whatever its FV
    // and ND.
    auto main_loop = [&](auto fv_const, auto nd_const) {
      constexpr int FV = decltype(fv_const)::value;
      constexpr int ND = decltype(nd_const)::value;
      auto dma = [&](int s) {
#pragma unroll
        for (int i = 0; i < ND; ++i) issue(i, s);
      };
      constexpr int NMEMV = FV + FW + ND;
      constexpr int QMV = (FW * FV) / NMEMV >= 2 ? 2 : 1;
      bf16x8_t fa0[FV], fw0[FW], fa1[FV], fw1[FW];
      auto read_stage = [&](int buf, bf16x8_t(&fa)[FV], bf16x8_t(&fw)[FW]) {
#pragma unroll
        for (int j = 0; j < FV; ++j) fa[j] = TM::read_a(As[buf], 0, j, wm);
#pragma unroll
        for (int i = 0; i < FW; ++i) fw[i] = TM::read_w(Ws[buf], i, wn);
      };
      auto iteration = [&](int s, bf16x8_t(&fa_cur)[FV], bf16x8_t(&fw_cur)[FW],
                           bf16x8_t(&fa_nxt)[FV], bf16x8_t(&fw_nxt)[FW]) {
        read_stage((s + 1) % NB, fa_nxt, fw_nxt);
#pragma unroll
        for (int i = 0; i < FW; ++i)
#pragma unroll
          for (int j = 0; j < FV; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fw_cur[i], fa_cur[j], acc[i][j],
                                                                 0, 0, 0);
        dma(s + 4);
        // operand reads one per QMV MFMAs, then the DMAs one per QMV MFMAs
        // (with too few MFMAs to spread them over, the compiler places them)
        if constexpr (QMV * NMEMV <= FW * FV) {
#pragma unroll
          for (int q = 0; q < FV + FW; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, QMV, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          }
#pragma unroll
          for (int q = 0; q < ND; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, QMV, 0);
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
          }
          if constexpr (FW * FV > QMV * NMEMV)
            __builtin_amdgcn_sched_group_barrier(0x008, FW * FV - QMV * NMEMV, 0);
        }
        // Stage s+2 has landed (stages s+3 and s+4 may still be in flight) and
        // this wave's operand reads are done; then a plain barrier (a fence
        // would also wait for the DMAs still in flight).  The empty asm
        // statements keep the compiler from moving LDS accesses across it.
        __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(2 * ND));
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
      };

      dma(0);
      dma(1);
      dma(2);
      dma(3);
      __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(2 * ND));   // stages 0 and 1
      __syncthreads();
      read_stage(0, fa0, fw0);
      // iteration 0 DMAs stage 4 into stage 0's buffer: every wave's reads of
      // stage 0 must be done first (later stages are read before the barrier
      // that ends the previous iteration)
      __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(63));
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");

      // two stages per trip so the register sets are named statically (nk is
      // even: K is a multiple of 64)
      for (int s = 0; s < nk; s += 2) {
        iteration(s, fa0, fw0, fa1, fw1);
        iteration(s + 1, fa1, fw1, fa0, fw0);
      }
    };
    if constexpr (TM::KN) {
      // k-row weights (2 x 4 waves, 8 fragments per wave): every fragment
      // is computed, which keeps fewer copies of the loop
      with_count0<BPW>(ndma, [&](auto ndc) { main_loop(IntC<FM>{}, ndc); });
    } else {
      // fragments j < fv of this wave hold rows below hv
      const int nfr = (t.hv + 15) / 16;
      const int fv = __builtin_amdgcn_readfirstlane(nfr > wm ? (nfr - wm + WM - 1) / WM : 0);
      with_count<FM>(fv, [&](auto fvc) {
        with_count0<BPW>(ndma, [&](auto ndc) { main_loop(fvc, ndc); });
      });
    }
    // the next tile's first DMAs (and the staged output) go to buffers that
    // the last (unused) DMAs and reads above may still touch
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __syncthreads();
    // staged stores: measured on MI355X 1-2 % faster for the SwiGLU up, the
    // down and the backward's k-row products; 7 % slower for the GELU up
    // projection of the GPT-2 shape (short K, 256-column tiles), which
    // keeps the direct stores
    if constexpr (mode_pre(MODE) || mode_gelu(MODE)) {
      TM::epilogue(a, t, acc, wm, wn);
    } else {
      TM::epilogue_staged(a, t, acc, wm, wn, ring);
      __syncthreads();   // the staged rows are read before the next DMAs
    }
  }
}

// The main loop of gemm_dma_kernel for one tile, taking the tile's stage
// count: k stages 0 .. nk-1 (nk even) of the operands behind t's
// descriptors, row stride row_bytes, into acc.  (The forward kernel keeps
// its own copy of this loop: folded into a function it compiled slower.)
template <int BM, int BNW, int WM, int WN, int MODE>
struct DmaLoop {
  static constexpr int BK = 32, NB = 4, NW = WM * WN;
  using TM = TileMath<BM, BNW, WM, WN, BK, MODE>;
  static constexpr int CH = TM::CH, FM = TM::FM, FW = TM::FW;
  static constexpr int ABLK = BM / 16, WBLK = BNW / 16;   // 16-row DMA blocks
  static constexpr int NBLK = ABLK + WBLK;
  // blocks per wave.  A wave whose first block is past the stage's last
  // (the eighth wave of a 192-row tile: 28 blocks for 8 waves of 4) issues
  // no DMAs: its vmcnt wait is then empty, and the barrier after it still
  // waits for every other wave's.  Were a wave's blocks only partly past
  // the end, it would repeat the stage's last block (same data to the same
  // place), so that its vmcnt counts stages like everyone else's.
  static constexpr int BPW = (NBLK + NW - 1) / NW;
  static_assert(CH == 4, "k32 stages");
  // interleave: QM MFMAs per operand read or DMA, then the rest
  static constexpr int NMEM = FM + FW + BPW;
  static constexpr int QM = (FW * FM) / NMEM >= 2 ? 2 : 1;
  static_assert(QM * NMEM <= FW * FM, "operand traffic fits the MFMA stream");

  static __device__ __forceinline__ void run(const Tile &t, int nk, uint32_t row_bytes,
                                             u32x4_t (*As)[BM * CH], u32x4_t (*Ws)[BNW * CH],
                                             int wave, int wm, int wn,
                                             f32x4_t (&acc)[FW][FM]) {
    const int lane = threadIdx.x % 64;
    // lane -> row lane / 4 of a 16-row block, the chunk its LDS slot holds
    const uint32_t voff = (uint32_t)(lane / 4) * row_bytes + dma32_chunk_bytes(lane);
    // wave w moves blocks BPW w .. BPW w + BPW - 1 of the stage: token
    // blocks first, then weight blocks (SwiGLU: gate rows from one
    // descriptor, up rows from the other)
    auto dma = [&](int s) {
      if (wave * BPW >= NBLK) return;
#pragma unroll
      for (int i = 0; i < BPW; ++i) {
        const int blk = min(wave * BPW + i, NBLK - 1);
        __amdgpu_buffer_rsrc_t rs;
        u32x4_t *dst;
        int row;
        if (blk < ABLK) {
          rs = t.rs_a;
          dst = As[s % NB] + blk * 64;
          row = blk * 16;
        } else {
          const int wb = blk - ABLK;
          dst = Ws[s % NB] + wb * 64;
          if (TM::SWI && wb >= WBLK / 2) {
            rs = t.rs_w1;
            row = (wb - WBLK / 2) * 16;
          } else {
            rs = t.rs_w0;
            row = wb * 16;
          }
        }
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 16, voff,
                                                 row * (int)row_bytes + s * (BK * 2), 0, 0);
      }
    };

    bf16x8_t fa0[FM], fw0[FW], fa1[FM], fw1[FW];
    auto read_stage = [&](int buf, bf16x8_t(&fa)[FM], bf16x8_t(&fw)[FW]) {
#pragma unroll
      for (int j = 0; j < FM; ++j) fa[j] = TM::read_a(As[buf], 0, j, wm);
#pragma unroll
      for (int i = 0; i < FW; ++i) fw[i] = TM::read_w(Ws[buf], i, wn);
    };
    auto iteration = [&](int s, bf16x8_t(&fa_cur)[FM], bf16x8_t(&fw_cur)[FW],
                         bf16x8_t(&fa_nxt)[FM], bf16x8_t(&fw_nxt)[FW]) {
      read_stage((s + 1) % NB, fa_nxt, fw_nxt);
#pragma unroll
      for (int i = 0; i < FW; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fw_cur[i], fa_cur[j], acc[i][j],
                                                               0, 0, 0);
      dma(s + 4);
      // operand reads one per QM MFMAs, then the DMAs one per QM MFMAs
#pragma unroll
      for (int q = 0; q < FM + FW; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, QM, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
#pragma unroll
      for (int q = 0; q < BPW; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, QM, 0);
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      }
      if constexpr (FW * FM > QM * NMEM)
        __builtin_amdgcn_sched_group_barrier(0x008, FW * FM - QM * NMEM, 0);
      // Stage s+2 has landed (stages s+3 and s+4 may still be in flight) and
      // this wave's operand reads are done; then a plain barrier (a fence
      // would also wait for the DMAs still in flight).  The empty asm
      // statements keep the compiler from moving LDS accesses across it.
      __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(2 * BPW));
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    };

    dma(0);
    dma(1);
    dma(2);
    dma(3);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(2 * BPW));   // stages 0 and 1
    __syncthreads();
    read_stage(0, fa0, fw0);
    // iteration 0 DMAs stage 4 into stage 0's buffer: every wave's reads of
    // stage 0 must be done first
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(63));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");

    // two stages per trip so the register sets are named statically (nk is
    // even)
    for (int s = 0; s < nk; s += 2) {
      iteration(s, fa0, fw0, fa1, fw1);
      iteration(s + 1, fa1, fw1, fa0, fw0);
    }
    // the next tile's first DMAs go to buffers that the last (unused) DMAs
    // and reads above may still touch
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __syncthreads();
  }
};

// ------------------------------------------------------ weight gradients --
// dW[g] = A_g^T B_g summed over the rows of group g (the backward pass of
// the grouped GEMMs), from K-contiguous transposed copies At [M, Rp] and Bt
// [N, Rp] whose group column ranges [poff[g], poff[g+1]) are zero-padded to
// multiples of 64:  out[g][m][n] = sum_j At[m][j] * Bt[n][j], accumulated in
// fp32 and rounded once to bf16 (the dtype of the weights).  The
// same tile arithmetic as the forward kernels with the group's rows as the
// contraction, k loop over the group's columns (none for an empty group:
// its tiles store zeros).
struct WgradArgs {
  const int32_t *poff;   // [G + 1], multiples of 64
  int G, Rp, M, N;
  const uint16_t *at;    // [M, Rp]
  const uint16_t *bt;    // [N, Rp]
  uint16_t *out;         // [G][M][N] bf16 (or [G - 1] when out_last is set)
  uint16_t *out_last;    // the last group's [M][N] stored apart, or NULL
  int m_tiles, n_tiles;
};

// Ids of the groups whose padded column count is above 64 (LONG) or at most
// 64, in group order, into list; returns their number.  Thread t looks at
// groups 2t and 2t+1 (G <= 2 * NT).
template <int NT, bool LONG>
__device__ __forceinline__ int wgrad_group_list(const int32_t *poff, int G, int *list,
                                                int *tmp) {
  static_assert(2 * NT >= kMaxExperts + 1, "two groups per thread cover E + S");
  int f[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int g = 2 * threadIdx.x + q;
    const int kc = g < G ? poff[g + 1] - poff[g] : -1;
    f[q] = g < G && (LONG ? kc > 64 : kc <= 64);
  }
  int total;
  const int ex = block_exclusive_scan<NT>(f[0] + f[1], tmp, &total);
  if (f[0]) list[ex] = 2 * threadIdx.x;
  if (f[1]) list[ex + f[0]] = 2 * threadIdx.x + 1;
  __syncthreads();
  return total;
}

// Persistent grid over the (group, m-tile, n-tile) space of the groups with
// more than 64 columns, in the slice order of the forward kernels; each tile
// runs the DMA-fed main loop over its group's columns (padded to 64, so the
// stage count is even) with the descriptors based at the group's first
// column.  Groups of at most 64 columns go to gemm_wgrad_short_kernel.
template <int BM, int BNW, int WM, int WN>
__global__ __launch_bounds__(WM *WN * 64) __attribute__((amdgpu_waves_per_eu(WM * WN / 4)))
void gemm_wgrad_kernel(WgradArgs a) {
  using DL = DmaLoop<BM, BNW, WM, WN, kDown>;
  using TM = typename DL::TM;
  constexpr int CH = TM::CH, NB = DL::NB, NT = TM::NT;
  constexpr int FM = TM::FM, FW = TM::FW, WTW = TM::WTW;
  // the operand buffers, reused after the main loop to stage the output
  // tile (BM rows of BNW bf16) so that it leaves in whole 16-byte chunks
  constexpr int LDS_CHUNKS = NB * (BM + BNW) * CH;
  static_assert(BM * BNW * 2 <= LDS_CHUNKS * 16, "output tile fits the operand buffers");
  constexpr int OCH = BNW / 8;   // 16-byte chunks per output row
  __shared__ u32x4_t lds[LDS_CHUNKS];
  auto As = reinterpret_cast<u32x4_t(*)[BM * CH]>(lds);
  auto Ws = reinterpret_cast<u32x4_t(*)[BNW * CH]>(lds + NB * BM * CH);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
  const int wm = wave / WN;
  const int wn = wave % WN;
  const int lane = threadIdx.x % 64;
  __shared__ int glist[kMaxExperts + 1];
  __shared__ int gtmp[NT / 64];
  const int ng = wgrad_group_list<NT, true>(a.poff, a.G, glist, gtmp);
  const int per_g = a.m_tiles * a.n_tiles;
  const int total = ng * per_g;
  const uint32_t row_bytes = (uint32_t)a.Rp * 2u;

  for (int it = 0;; ++it) {
    const int L = slice_tile(it);
    if (L >= total) break;
    const int g = glist[L / per_g];
    const int local = L % per_g;
    Tile t;
    t.g = g;
    t.gather = false;
    t.grow0 = 0;
    t.rows = a.M;
    t.m0 = (local % a.m_tiles) * BM;
    t.hv = min(BM, a.M - t.m0);
    t.n0 = (local / a.m_tiles) * BNW;
    const int c0 = __builtin_amdgcn_readfirstlane(a.poff[g]);
    const int c1 = __builtin_amdgcn_readfirstlane(a.poff[g + 1]);
    const int nk = c1 > c0 ? (c1 - c0) / 32 : 0;
    const int arows = min(BM, a.M - t.m0);
    const int wrows = min(BNW, a.N - t.n0);
    t.rs_a = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(a.at + (int64_t)t.m0 * a.Rp + c0), 0, arows * row_bytes, kBufferWord3);
    t.rs_w0 = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(a.bt + (int64_t)t.n0 * a.Rp + c0), 0, wrows * row_bytes, kBufferWord3);
    t.rs_w1 = t.rs_w0;

    f32x4_t acc[FW][FM];
#pragma unroll
    for (int i = 0; i < FW; ++i)
#pragma unroll
      for (int j = 0; j < FM; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    DL::run(t, nk, row_bytes, As, Ws, wave, wm, wn, acc);

    // lane owns columns 4*(lane/16)+0..3 of row lane%16 of each fragment:
    // 8 bytes into the staged tile, whose 16-byte chunks are XOR-swizzled by
    // row (chunk c of row r at c ^ (r & 7)) to spread a fragment's 16 rows
    // over the banks
    char *st = reinterpret_cast<char *>(lds);
#pragma unroll
    for (int i = 0; i < FW; ++i) {
      const int col = wn * WTW + i * 16 + 4 * (lane / 16);
#pragma unroll
      for (int j = 0; j < FM; ++j) {
        const int r = TM::frag_row(wm, j) + lane % 16;
        uint2 v;
        v.x = pack_bf16x2(acc[i][j][0], acc[i][j][1]);
        v.y = pack_bf16x2(acc[i][j][2], acc[i][j][3]);
        *reinterpret_cast<uint2 *>(st + r * (BNW * 2) + (((col >> 3) ^ (r & 7)) << 4) +
                                   (col & 7) * 2) = v;
      }
    }
    __syncthreads();
    uint16_t *o = (a.out_last && g == a.G - 1) ? a.out_last : a.out + (int64_t)g * a.M * a.N;
#pragma unroll
    for (int q = threadIdx.x; q < BM * OCH; q += NT) {
      const int r = q / OCH, c = q % OCH;
      const u32x4_t v = lds[r * OCH + (c ^ (r & 7))];
      // streaming stores: the gradient is not read again here (measured:
      // plain stores wrote it at about 2.5 TB/s)
      if (t.m0 + r < a.M && t.n0 + 8 * c < a.N)
        __builtin_nontemporal_store(
            v, reinterpret_cast<u32x4_t *>(o + (int64_t)(t.m0 + r) * a.N + t.n0 + 8 * c));
    }
    // the next tile's first DMAs overwrite the staged tile
    __syncthreads();
  }
}

// Weight gradients of the groups with at most 64 columns (cold experts:
// the contraction is one or two k32 steps, the cost is writing the M x N
// output).  BM x BN tiles (launched as 128 x 128), four waves of 64 x 64;
// the operand fragments come straight from global memory (no operand
// pipeline to fill) and several workgroups per CU hide the latency.  The
// N-side fragment is the MFMA's A operand so that a lane ends with 4
// consecutive output columns of one row; the tile is staged in LDS (16-byte
// chunks XOR-swizzled by row) and leaves in whole 16-byte chunks with
// streaming stores, a row's 256 bytes per 16 threads.  A group without rows
// gets zeros.  Measured on an all-cold batch at the DeepSeek-V3 dimensions:
// the W_up gradient in 4.8 ms against 6.1 ms in the DMA-fed kernel.
template <int BM, int BN>
__global__ __launch_bounds__(256) void gemm_wgrad_short_kernel(WgradArgs a) {
  __shared__ int glist[kMaxExperts + 1];
  __shared__ int gtmp[4];
  constexpr int OCH = BN / 8;   // 16-byte chunks per output row
  __shared__ u32x4_t st[BM * OCH];
  const int ng = wgrad_group_list<256, false>(a.poff, a.G, glist, gtmp);
  static_assert((BM / 64) * (BN / 64) == 4, "four waves of 64 x 64");
  const int lane = threadIdx.x % 64;
  const int wave = threadIdx.x / 64;
  const int wm = wave / (BN / 64), wn = wave % (BN / 64);
  const int mt = (a.M + BM - 1) / BM, nt = (a.N + BN - 1) / BN;
  const int per_g = mt * nt;
  const int total = ng * per_g;
  const int lr = lane % 16, lk = 8 * (lane / 16);
  for (int L = blockIdx.x; L < total; L += gridDim.x) {
    const int g = glist[L / per_g];
    const int local = L % per_g;
    // n-tile fastest: the workgroups in flight together write whole output
    // rows (contiguous memory) rather than 256-byte pieces of many rows
    const int tm0 = (local / nt) * BM, tn0 = (local % nt) * BN;
    const int m0 = tm0 + wm * 64;
    const int n0 = tn0 + wn * 64;
    const int c0 = a.poff[g];
    const int ksteps = (a.poff[g + 1] - c0) / 32;
    f32x4_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int ks = 0; ks < ksteps; ++ks) {
      const int col = c0 + 32 * ks + lk;
      bf16x8_t fn[4], fm[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int n = n0 + 16 * i + lr;
        const int m = m0 + 16 * i + lr;
        fn[i] = n < a.N ? *reinterpret_cast<const bf16x8_t *>(a.bt + (int64_t)n * a.Rp + col)
                        : bf16x8_t{};
        fm[i] = m < a.M ? *reinterpret_cast<const bf16x8_t *>(a.at + (int64_t)m * a.Rp + col)
                        : bf16x8_t{};
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fn[i], fm[j], acc[i][j], 0, 0, 0);
    }
    // stage: row r (tile-local m), column c (tile-local n) at chunk
    // (c / 8) ^ (r & 7) of row r
    char *sb = reinterpret_cast<char *>(st);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = wn * 64 + 16 * i + 4 * (lane / 16);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = wm * 64 + 16 * j + lr;
        uint2 v;
        v.x = pack_bf16x2(acc[i][j][0], acc[i][j][1]);
        v.y = pack_bf16x2(acc[i][j][2], acc[i][j][3]);
        *reinterpret_cast<uint2 *>(sb + r * (BN * 2) + (((c >> 3) ^ (r & 7)) << 4) + (c & 7) * 2) = v;
      }
    }
    __syncthreads();
    uint16_t *o = (a.out_last && g == a.G - 1) ? a.out_last : a.out + (int64_t)g * a.M * a.N;
#pragma unroll
    for (int q = threadIdx.x; q < BM * OCH; q += 256) {
      const int r = q / OCH, c = q % OCH;
      const u32x4_t v = st[r * OCH + (c ^ (r & 7))];
      if (tm0 + r < a.M && tn0 + 8 * c < a.N)
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t *>(o + (int64_t)(tm0 + r) * a.N +
                                                                   tn0 + 8 * c));
    }
    __syncthreads();   // the next tile's staging overwrites st
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

// Persistent launch: one resident wave of workgroups walks all tiles (fewer
// when there are fewer tiles), rounded to a multiple of 8 for the slice
// order.  `per_cu` caches the occupancy of the instantiation.
template <int BM, int BN_OUT, int NT>
static hipError_t launch_persistent(const void *kernel, int &per_cu, GemmArgs a,
                                    hipStream_t s) {
  a.n_tiles = (a.n_out + BN_OUT - 1) / BN_OUT;
  // upper bound of the ragged m-tile count: every group wastes < 1 tile
  const int64_t mt_bound = (int64_t)(a.routed_rows + BM - 1) / BM + a.E + a.S;
  const int64_t tiles = mt_bound * a.n_tiles;
  if (!per_cu) {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kernel, NT, 0) != hipSuccess || nb <= 0)
      nb = 1;
    per_cu = nb;
  }
  int64_t grid = (int64_t)num_cus() * per_cu;
  if (tiles < grid) grid = tiles;
  grid = ((grid + 7) / 8) * 8;
  void *args[] = {&a};
  return hipLaunchKernel(kernel, dim3((unsigned)grid), dim3(NT), args, 0, s);
}

template <int BM, int BNW, int WM, int WN, int BK, int PFD, int MODE, bool WT>
static hipError_t launch_bm(const GemmArgs &a, hipStream_t s) {
  static int per_cu = 0;
  return launch_persistent<BM, mode_swiglu(MODE) ? BNW / 2 : BNW, WM * WN * 64>(
      reinterpret_cast<const void *>(&gemm_bf16_kernel<BM, BNW, WM, WN, BK, PFD, MODE, WT>),
      per_cu, a, s);
}

template <int BM, int MODE>
static hipError_t launch_pp(const GemmArgs &a, hipStream_t s) {
  static int per_cu = 0;
  return launch_persistent<BM, mode_swiglu(MODE) ? 128 : 256, 512>(
      reinterpret_cast<const void *>(&gemm_pp_kernel<BM, MODE>), per_cu, a, s);
}

template <int BM, int BNW, int WM, int WN, int MODE, bool WT>
static hipError_t launch_dma(const GemmArgs &a, hipStream_t s) {
  static int per_cu = 0;
  return launch_persistent<BM, mode_swiglu(MODE) ? BNW / 2 : BNW, WM * WN * 64>(
      reinterpret_cast<const void *>(&gemm_dma_kernel<BM, BNW, WM, WN, MODE, WT>), per_cu, a,
      s);
}

// Large groups.  Row tile: 256 or 192 token rows, whichever needs fewer
// tile rounds over the persistent grid (one workgroup per CU) once the
// smaller tile's lower operand reuse is priced in (measured: about 12 %
// more time per row); group sizes are device-side, so the count of m-tiles
// is estimated as rows / BM plus half a tile per group.  Kernel: the
// DMA-fed one, except row-major weights with K > 8192, which take the
// ping-pong one (measured on MI355X: at K = 14336 the ping-pong kernel wins
// over row-major weights, the DMA-fed one over tiled weights).
template <int MODE, bool WT>
static hipError_t launch_big(const GemmArgs &a, hipStream_t s) {
  const double nblk = num_cus();
  const int bn_out = mode_swiglu(MODE) ? 128 : 256;
  const double n_tiles = (a.n_out + bn_out - 1) / bn_out;
  const double rows = (double)a.routed_rows + (double)a.S * a.T;
  const double groups = a.E + a.S;
  auto cost = [&](double bm, double per_row) {
    const double mt = rows / bm + 0.5 * groups;
    return std::ceil(mt * n_tiles / nblk) * bm * per_row;
  };
  const bool bm192 = cost(192, 1.12) < cost(256, 1.0);
  // k-row weights: waves of 128 (96) token rows x 64 weight rows, so that
  // each wave makes fewer of the (twice as many) transposing weight reads
  if constexpr (mode_kn(MODE)) {
    return bm192 ? launch_dma<192, 256, 2, 4, MODE, WT>(a, s)
                 : launch_dma<256, 256, 2, 4, MODE, WT>(a, s);
  } else {
    if constexpr (!WT) {
      if (a.K > 8192) return bm192 ? launch_pp<192, MODE>(a, s) : launch_pp<256, MODE>(a, s);
    }
    return bm192 ? launch_dma<192, 256, 4, 2, MODE, WT>(a, s)
                 : launch_dma<256, 256, 4, 2, MODE, WT>(a, s);
  }
}

// Groups are split by row count into tile classes, one launch each: small
// groups (<= 64 rows: decode batches, cold experts) stream their weights
// through 32- or 64-row tiles; larger groups use 256- or 192-row tiles.  The
// large class is skipped when no group can exceed 64 rows (every group has
// at most T rows); the small classes when groups are large on average.
template <int MODE, bool WT>
static hipError_t launch_classes_t(GemmArgs a, hipStream_t s) {
  hipError_t err = hipSuccess;
  // Groups average 512 rows or more: small groups are rare enough that the
  // large-tile launch takes every group and the second launch is saved.
  if ((int64_t)a.routed_rows >= 512ll * a.E) {
    a.min_rows = 1;
    a.max_rows = 1 << 30;
    return launch_big<MODE, WT>(a, s);
  }
  if (a.T > 64) {
    a.min_rows = 65;
    a.max_rows = 1 << 30;
    if ((err = launch_big<MODE, WT>(a, s)) != hipSuccess) return err;
  }
  a.min_rows = 1;
  a.max_rows = 64;
  // Groups average 16 rows or more (cold experts of a large batch): those
  // of 33-64 rows take one 64-row tile, so each weight tile crosses the
  // load path once instead of twice (measured 1.2 % faster on a 256-expert
  // batch of 8192 tokens), with 8 waves of 16 x 64 (0.6 % faster than 4
  // waves of 32 x 64); decode batches keep the single launch.
  if ((int64_t)a.routed_rows >= 16ll * a.E) {
    a.min_rows = 33;
    if ((err = launch_bm<64, 128, 4, 2, 64, 2, MODE, WT>(a, s)) != hipSuccess) return err;
    a.min_rows = 1;
    a.max_rows = 32;
  }
  return launch_bm<32, 128, 2, 2, 64, 2, MODE, WT>(a, s);
}

// The kernels compiled for the weights' order (k-row weights: row-major only).
template <int MODE>
static hipError_t launch_classes(const GemmArgs &a, hipStream_t s) {
  if constexpr (!mode_kn(MODE)) {
    if (a.w_tiled) return launch_classes_t<MODE, true>(a, s);
  }
  return launch_classes_t<MODE, false>(a, s);
}

// Plain grouped linear map c[r] = a[r] W[g]^T (+ bias[g]) over the groups of
// `offsets` and the shared group (rows T*k.., operand a_shared, weights
// w_shared), each W[g] stored [n_out][K] or (w_kn) [K][n_out]: the backward
// pass's dH = dY W2 and dX = dA W1 (k-row weights as stored) and the
// pre-activation recomputation A = X W1^T.
hipError_t launch_grouped_linear_bf16(const int32_t *offsets, int E, int S, int T, int k,
                                      int K, int n_out, const void *a_routed,
                                      const void *a_shared, const void *w,
                                      const void *w_shared, const void *bias, void *c,
                                      bool w_kn, hipStream_t s) {
  GemmArgs a{};
  a.offsets = offsets;
  a.E = E;
  a.S = S;
  a.T = T;
  a.routed_rows = T * k;
  a.a_routed = static_cast<const uint16_t *>(a_routed);
  a.a_shared = static_cast<const uint16_t *>(a_shared);
  a.K = K;
  a.w = static_cast<const uint16_t *>(w);
  a.w_shared = static_cast<const uint16_t *>(w_shared);
  a.w_rows = n_out;
  a.bias = static_cast<const uint16_t *>(bias);
  a.c = static_cast<uint16_t *>(c);
  a.n_out = n_out;
  return w_kn ? launch_classes<kDownKN>(a, s) : launch_classes<kDown>(a, s);
}

hipError_t launch_wgrad_bf16(const int32_t *poff, int G, int Rp, int M, int N, const void *at,
                             const void *bt, void *out, void *out_last, hipStream_t s) {
  constexpr int BM = 256, BNW = 256;
  WgradArgs a{};
  a.poff = poff;
  a.G = G;
  a.Rp = Rp;
  a.M = M;
  a.N = N;
  a.at = static_cast<const uint16_t *>(at);
  a.bt = static_cast<const uint16_t *>(bt);
  a.out = static_cast<uint16_t *>(out);
  a.out_last = static_cast<uint16_t *>(out_last);
  a.m_tiles = (M + BM - 1) / BM;
  a.n_tiles = (N + BNW - 1) / BNW;
  static int per_cu = 0;
  const void *kern = reinterpret_cast<const void *>(&gemm_wgrad_kernel<BM, BNW, 4, 2>);
  if (!per_cu) {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kern, 512, 0) != hipSuccess || nb <= 0)
      nb = 1;
    per_cu = nb;
  }
  int64_t grid = (int64_t)num_cus() * per_cu;
  const int64_t tiles = (int64_t)G * a.m_tiles * a.n_tiles;
  if (tiles < grid) grid = tiles;
  grid = ((grid + 7) / 8) * 8;
  void *args[] = {&a};
  hipError_t err = hipLaunchKernel(kern, dim3((unsigned)grid), dim3(512), args, 0, s);
  if (err != hipSuccess) return err;
  // the groups of at most 64 columns (the split is device-side: each
  // kernel takes its own groups from poff)
  constexpr int SBM = 128, SBN = 128;
  static int per_cu_short = 0;
  const void *kshort = reinterpret_cast<const void *>(&gemm_wgrad_short_kernel<SBM, SBN>);
  if (!per_cu_short) {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kshort, 256, 0) != hipSuccess ||
        nb <= 0)
      nb = 1;
    per_cu_short = nb;
  }
  const int64_t stiles = (int64_t)G * ((M + SBM - 1) / SBM) * ((N + SBN - 1) / SBN);
  const int64_t sgrid = std::min<int64_t>(stiles, (int64_t)num_cus() * per_cu_short);
  return hipLaunchKernel(kshort, dim3((unsigned)sgrid), dim3(256), args, 0, s);
}

hipError_t launch_expert_up_bf16(bool swiglu, const int32_t *offsets, int E, int S,
                                 int T, int k, int d, int h, const void *x_perm,
                                 const int32_t *perm_src, const void *x, const void *w_up,
                                 const void *w_up_shared, const void *b_up,
                                 void *hidden, bool w_tiled, hipStream_t s) {
  GemmArgs a{};
  a.w_tiled = w_tiled;
  if (!x_perm) {   // token rows gathered from x
    a.gather = perm_src;
    a.gather_x = static_cast<const uint16_t *>(x);
  }
  a.offsets = offsets;
  a.E = E;
  a.S = S;
  a.T = T;
  a.routed_rows = T * k;
  // (gathered rows: a_routed only stands in for the unused grouped copy)
  a.a_routed = static_cast<const uint16_t *>(x_perm ? x_perm : x);
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

// The up projection of a training step: hidden as above, and the
// pre-activations [rows, w_rows] (SwiGLU gate rows then up rows; GELU with
// the bias) that the backward pass differentiates through.
hipError_t launch_expert_up_train_bf16(bool swiglu, const int32_t *offsets, int E, int S,
                                       int T, int k, int d, int h, const void *x_perm,
                                       const int32_t *perm_src, const void *x,
                                       const void *w_up, const void *w_up_shared,
                                       const void *b_up, void *hidden, void *preact,
                                       bool w_tiled, hipStream_t s) {
  GemmArgs a{};
  a.w_tiled = w_tiled;
  if (!x_perm) {   // token rows gathered from x
    a.gather = perm_src;
    a.gather_x = static_cast<const uint16_t *>(x);
  }
  a.offsets = offsets;
  a.E = E;
  a.S = S;
  a.T = T;
  a.routed_rows = T * k;
  a.a_routed = static_cast<const uint16_t *>(x_perm ? x_perm : x);
  a.a_shared = static_cast<const uint16_t *>(x);
  a.K = d;
  a.w = static_cast<const uint16_t *>(w_up);
  a.w_shared = static_cast<const uint16_t *>(w_up_shared);
  a.w_rows = swiglu ? 2 * h : h;
  a.bias = static_cast<const uint16_t *>(b_up);
  a.c = static_cast<uint16_t *>(hidden);
  a.n_out = h;
  a.c_pre = static_cast<uint16_t *>(preact);
  return swiglu ? launch_classes<kUpSwigluPre>(a, s) : launch_classes<kUpGeluPre>(a, s);
}

hipError_t launch_expert_down_bf16(const int32_t *offsets, int E, int S, int T,
                                   int k, int d, int h, const void *hidden,
                                   const void *w_down, const void *w_down_shared,
                                   const void *b_down, void *y_perm,
                                   bool w_tiled, hipStream_t s) {
  GemmArgs a{};
  a.w_tiled = w_tiled;
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

// Tiled weight order (GemmArgs::w_tiled) of a [rows, cols] bf16 matrix
// stack: 16-byte piece q of dst lies in block b = q / 64 = (rb, kb), rb =
// b / (cols/32), kb = b % (cols/32), at p = q % 64, and holds row 16 rb +
// p / 4, columns 32 kb + 8 c .. + 7 with c = (p % 4) ^ (p / 16): the LDS
// order of a 16-row k32 block of the DMA-fed kernel.  One thread per piece,
// consecutive threads writing consecutive pieces.
__global__ __launch_bounds__(256) void tile_weights_kernel(const u32x4_t *__restrict__ src,
                                                           u32x4_t *__restrict__ dst,
                                                           int64_t pieces, int nkb) {
  for (int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x; q < pieces;
       q += (int64_t)gridDim.x * 256) {
    const int64_t b = q / 64;
    const int p = (int)(q % 64);
    const int64_t row = (b / nkb) * 16 + p / 4;
    const int c = (p % 4) ^ (p / 16);
    dst[q] = src[row * (4 * nkb) + (b % nkb) * 4 + c];
  }
}

hipError_t launch_tile_weights(const void *src, void *dst, int64_t rows, int cols,
                               hipStream_t s) {
  const int64_t pieces = rows * (cols / 8);
  if (pieces == 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((pieces + 255) / 256, 8192);
  tile_weights_kernel<<<dim3((unsigned)blocks), dim3(256), 0, s>>>(
      static_cast<const u32x4_t *>(src), static_cast<u32x4_t *>(dst), pieces, cols / 32);
  return hipGetLastError();
}

}  // namespace moe
