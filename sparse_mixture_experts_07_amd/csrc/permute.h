// permute.h - host interface of the dispatch kernels (permute.hip).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace moe {

int perm_num_segments(int64_t n);

// Stable grouping of the T*k assignments idx (ids outside [0, E) are left
// out), an expert keeping its first `capacity` (0: all) in flat order; then
// the row move into x_perm (skipped when x_perm is NULL).  importance NULL:
// no Importance and no statistics.  counts_out (or NULL): the assignments
// per expert (every one, the router's count).  hist [nseg * E],
// full_off [E + 1] and perm_w [T*k] are scratch.
hipError_t launch_permute(const int32_t *idx, const float *w, const void *x, int T, int k,
                          int E, int capacity, int row_bytes, int32_t *offsets,
                          int32_t *perm_src, int32_t *pos, float *importance, double *stats,
                          void *x_perm, int32_t *hist, int32_t *full_off, float *perm_w,
                          hipStream_t s, int32_t *counts_out = nullptr);

// Scratch of the next-choice re-routing: T*k int32 each for pos_a, cand,
// pos_b and fin; E + 1 int32 each for off_b and full_off_b.
struct RerouteScratch {
  int32_t *pos_a, *cand, *pos_b, *fin, *off_b, *full_off_b;
};

// launch_permute under a capacity with the overflow re-routed one hop to the
// next choice (logits [T, E]: the scores the top k was taken on).
hipError_t launch_permute_reroute(const int32_t *idx, const float *w, const float *logits,
                                  const void *x, int T, int k, int E, int capacity,
                                  int row_bytes, int32_t *offsets, int32_t *perm_src,
                                  int32_t *pos, float *importance, double *stats,
                                  void *x_perm, int32_t *hist, int32_t *full_off,
                                  float *perm_w, const RerouteScratch &r, hipStream_t s,
                                  int32_t *counts_out = nullptr);

// The allocation-free dispatch's scratch: a static device array of this
// many bytes per GPU; noalloc_scratch() gives the current device's address
// (taken with hipGetSymbolAddress on the first call on each device).
constexpr size_t kNoallocScratchBytes = size_t(64) << 20;
hipError_t noalloc_scratch(void **ptr);

}  // namespace moe
