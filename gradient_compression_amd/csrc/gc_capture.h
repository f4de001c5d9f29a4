// gc_capture.h -- device helpers shared by the streaming pass (gc_pass.hip) and the kernels
// after it (gc_topk.hip): a segment's capture threshold, tile geometry, the capture of one
// tile's run of candidates, and the reset of the per-call lists.
#pragma once
#include "gc_device.h"

namespace gc {
namespace {

// Capture threshold of segment s in this call: the Top-k estimate, the Random-k plan
// threshold, or for a threshold call max(key(|tau|), floor), the floor being the estimate of
// the k-th largest key kept from the last threshold calls (so the capture stays within its
// capacity when more than k entries reach tau).  Small segments capture nothing.
__device__ __forceinline__ uint32_t capture_thr(const DevPlan& P, int s) {
  if (P.codec != kCodecThreshold) return P.thr[s];
  if (P.seg_flags[s] & kSegSmall) return kNoCapture;
  const uint32_t tk = mag_key(P.tau[s]), fl = P.thr_est[s];
  return fl == kNoCapture ? tk : max(tk, fl);
}

// Tile t of segment s: first element and length.
__device__ __forceinline__ void tile_range(const DevPlan& P, int s, int64_t t, int64_t* start,
                                           int* len) {
  const int64_t st = P.seg_off[s] + (t - P.tile_base[s]) * (int64_t)kTile;
  const int64_t rem = P.seg_off[s + 1] - st;
  *start = st;
  *len = rem < kTile ? (int)rem : kTile;
}

// Capture, in index order, the elements of tile t (values acc in the tile layout) whose key
// reaches thr: one atomic on the segment's counter (*count) reserves the tile's run; entries
// past the capacity are counted but not stored (the segment then leaves the candidate path).
__device__ __forceinline__ void capture_tile(const DevPlan& P, int s, int64_t t, int64_t start,
                                             int len, const f4 (&acc)[kSlots], uint32_t thr,
                                             uint32_t* count, uint32_t* s_w, uint32_t* s_base) {
  const int pb = slot_base();
  uint32_t bits[kSlots];
#pragma unroll
  for (int v = 0; v < kSlots; ++v) {
    uint32_t b = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c)
      b |= (pb + v * 256 + c < len && mag_key(acc[v][c]) >= thr) ? (1u << c) : 0u;
    bits[v] = b;
  }
  uint32_t woff[kSlots];
  const uint32_t total = tile_rank(bits, woff, s_w);
  if (threadIdx.x == 0) {
    const uint32_t base = total ? atomicAdd(count, total) : 0u;
    P.run_off[t] = base;
    P.run_cnt[t] = total;
    *s_base = base;
  }
  __syncthreads();
  if (total == 0) return;
  const uint32_t base = *s_base, cap = P.cand_cap[s];
  float* cv = P.cand_val + P.cand_base[s];
  int32_t* ci = P.cand_idx + P.cand_base[s];
  const int32_t lbase = (int32_t)(start - P.seg_off[s]) + pb;
#pragma unroll
  for (int v = 0; v < kSlots; ++v) {
    const uint32_t b = bits[v];
    if (!b) continue;
    uint32_t q = base + woff[v];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if ((b >> c) & 1u) {
        if (q < cap) {
          cv[q] = acc[v][c];
          ci[q] = lbase + v * 256 + c;
        }
        ++q;
      }
    }
  }
}

// The call's lists and the error flag start empty: cleared by the first workgroup of the
// streaming pass (the kernels that fill them run after it; the last call's readers have ended).
__device__ __forceinline__ void reset_call_lists(const DevPlan& P) {
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    *P.pend_count = 0;
    *P.act_count = 0;
    *P.full_count = 0;
    *P.err = 0;
  }
}

}  // namespace
}  // namespace gc
