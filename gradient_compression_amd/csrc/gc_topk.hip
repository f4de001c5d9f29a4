// gc_topk.hip -- gfx950 kernels of the error-feedback Top-k path after the streaming pass, and
// the threshold and Random-k sparsifiers that share its select and ordered emission.
//
// Top-k call (one stream, no host round trip; nine launches on a warm plan, two when every
// segment is modest: the pass, then k_single):
//   ef_capture  (gc_pass.hip) the streaming pass over g, e (and u): momentum, EF add, acc
//               written into e, and every (acc, index) whose magnitude key reaches the
//               segment's threshold captured, as one index-ordered run per tile [HBM-bound]
//   list        per segment: its path (candidates complete, small, or pending), the places
//               of its runs in index order, its candidate chunks listed.  Its other
//               workgroups run fb_hist:
//   fb_hist     \   only for pending segments (too few or too many candidates, or no
//   fb_capture   |  threshold yet); they end at once when none is pending: first-digit
//   fb_hist2     |  histogram of e, then a re-capture at the exact bucket floor, or (a bucket
//   fb_count    /   larger than the capacity) the radix select over the whole segment
//   scatter     candidates into ascending index order; a histogram of their keys in bins
//               that start at the capture threshold (two binades wide)
//   collect     per chunk: keys above the bin that holds the k-th key, and the keys inside
//               it appended to the segment's near list
//   finish      one workgroup per segment: the exact k-th key from the near list (in LDS),
//               the per-chunk offsets of the ordered emission, the next threshold estimate
//   emit        order-preserving compaction: keys above the k-th, then the ties in index
//               order; writes (value, index) and zeroes e (and u) where kept.  Small
//               segments are selected and emitted whole by workgroups of the same launch.
//
// Threshold and Random-k calls run the same select and emit on a per-call copy of the plan
// (their own k and capture threshold); Random-k ranks per-element Philox keys instead of
// magnitudes.  The two-pass codecs are in gc_codecs.hip, the payload scatters (int8 stage,
// decompression) in gc_scatter.hip, the shared device helpers in gc_device.h and
// gc_capture.h.
//
// The method is the Top-K with error feedback of "Communication Optimization > Gradient
// Compression" (Top-K section equations); momentum correction per the "Gradient
// Sparsification" glossary; the int8 stage per the "Gradient Compression" glossary
// (Top-k then 8-bit) with stochastic rounding (QSGD paragraph) and one scale per layer.
#include "gc_capture.h"
#include "gc_random.h"

#pragma clang fp contract(off)

namespace gc {
namespace {

__global__ __launch_bounds__(kThreads) void k_reset(DevPlan P) {
  const int s = blockIdx.x * kThreads + threadIdx.x;
  if (s < P.n_seg) {   // as on a fresh plan: no estimate, first margins
    P.thr[s] = P.thr_init[s];
    P.thr_est[s] = kNoCapture;
    P.beta[s] = kInitialBeta;
    P.beta_est[s] = kInitialBeta;
  }
}

// ------------------------------------------------------------------- per-call segment state
// Entries segment s keeps in this call: the plan's k, or for a threshold call the number of
// keys at or above key(|tau_s|) when that is smaller (the plan's k is then a cap).
__device__ __forceinline__ uint32_t call_k(const DevPlan& P, int s) {
  const uint32_t k = P.k[s];
  return P.codec == kCodecThreshold ? min(P.tau_cnt[s], k) : k;
}

// True when the streaming pass's capture does not hold segment s's k largest keys (fewer
// than k candidates, more than the capacity, or no threshold yet), so the fallback kernels
// re-capture it or select it over the whole segment.  Small segments and k = 0 never are.
__device__ __forceinline__ bool seg_pending(const DevPlan& P, int s) {
  if (P.seg_flags[s] & kSegSmall) return false;
  const uint32_t k = call_k(P, s);
  if (k == 0) return false;
  if (P.flags & kFlagForceFull) return true;
  const uint32_t c = P.cand_cnt[s];
  return capture_thr(P, s) == kNoCapture || c < k || c > P.cand_cap[s];
}

// ------------------------------------------------------------------------ digit histograms
__device__ __forceinline__ int digit_shift(int pass) { return pass == 0 ? 20 : (pass == 1 ? 9 : 0); }
__device__ __forceinline__ uint32_t digit_mask(int pass) { return pass == 2 ? 0x1FFu : 0x7FFu; }
__device__ __forceinline__ uint32_t prefix_mask(int pass) {
  return pass == 0 ? 0u : (pass == 1 ? 0x7FF00000u : 0x7FFFFE00u);
}
__device__ __forceinline__ uint32_t* seg_hist(const DevPlan& P, int s, int pass) {
  return P.hist + ((size_t)s * 3 + pass) * kHistBins;
}

// Add the keys of one tile-shaped block of values into the LDS histogram.
__device__ __forceinline__ void hist_add(uint32_t* h, const f4 (&x)[kSlots], int len,
                                         uint32_t prefix, int pass) {
  const int pb = slot_base(), sh = digit_shift(pass);
  const uint32_t pm = prefix_mask(pass), dm = digit_mask(pass);
#pragma unroll
  for (int v = 0; v < kSlots; ++v)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t key = mag_key(x[v][c]);
      if (pb + v * 256 + c < len && (key & pm) == prefix) atomicAdd(&h[(key >> sh) & dm], 1u);
    }
}

__device__ __forceinline__ void hist_flush(const uint32_t* h, uint32_t* gh) {
  for (int i = threadIdx.x; i < kHistBins; i += kThreads) {
    const uint32_t n = h[i];
    if (n) atomicAdd(&gh[i], n);
  }
}

// One digit's histogram of tile t of segment s (keys read from e, or Random-k keys), added
// into the segment's global histogram.  Contains barriers.
__device__ void hist_tile(const DevPlan& P, const float* __restrict__ e, int s, int64_t t,
                          uint32_t prefix, int pass, uint32_t* h) {
  int64_t start;
  int len;
  tile_range(P, s, t, &start, &len);
  for (int i = threadIdx.x; i < kHistBins; i += kThreads) h[i] = 0;
  f4 x[kSlots];
  key_tile(P, e, start, len, x);
  __syncthreads();
  hist_add(h, x, len, prefix, pass);
  __syncthreads();
  hist_flush(h, seg_hist(P, s, pass));
  __syncthreads();
}

// This thread's share of a histogram's bins, in descending bin order.
struct Bins {
  uint32_t v[kHistBins / kThreads];
};

__device__ __forceinline__ Bins load_bins(const uint32_t* gh) {
  Bins b;
#pragma unroll
  for (int j = 0; j < kHistBins / kThreads; ++j)
    b.v[j] = gh[kHistBins - 1 - (threadIdx.x * (kHistBins / kThreads) + j)];
  return b;
}

// Digit of the k-th largest key in a histogram of kHistBins bins (descending scan; each thread
// holds its share, load_bins): the bin d that holds it, the count above it and the bin's
// count.  s_tmp: __shared__ uint32_t[kWaves]; s_out: __shared__ uint32_t[3].  Contains
// barriers: call from every thread.
__device__ __forceinline__ bool find_digit_in(const Bins& b, uint32_t kk, uint32_t* s_tmp, uint32_t* s_out,
                              uint32_t* d_out, uint32_t* above_out, uint32_t* bin_out) {
  constexpr int kPer = kHistBins / kThreads;
  uint32_t sum = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) sum += b.v[j];
  if (threadIdx.x == 0) {
    s_out[0] = 0xFFFFFFFFu;
    s_out[1] = 0;
    s_out[2] = 0;
  }
  uint32_t tot;
  uint32_t acc = block_excl_scan<kThreads>(sum, s_tmp, &tot);
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    if (acc < kk && acc + b.v[j] >= kk) {
      s_out[0] = kHistBins - 1 - (threadIdx.x * kPer + j);
      s_out[1] = acc;
      s_out[2] = b.v[j];
    }
    acc += b.v[j];
  }
  __syncthreads();
  *d_out = s_out[0];
  *above_out = s_out[1];
  *bin_out = s_out[2];
  __syncthreads();   // s_out may be written again by the next call
  return *d_out != 0xFFFFFFFFu;
}

// find_digit_in over the histogram at gh (LDS or global).  kClear: each thread zeroes the bins
// it read, leaving the histogram clear for the next pass.  Contains barriers.
template <bool kClear = false>
__device__ bool find_digit(uint32_t* gh, uint32_t kk, uint32_t* s_tmp, uint32_t* s_out,
                           uint32_t* d_out, uint32_t* above_out, uint32_t* bin_out) {
  const Bins b = load_bins(gh);
  if (kClear) {
#pragma unroll
    for (int j = 0; j < kHistBins / kThreads; ++j)
      gh[kHistBins - 1 - (threadIdx.x * (kHistBins / kThreads) + j)] = 0;
  }
  return find_digit_in(b, kk, s_tmp, s_out, d_out, above_out, bin_out);
}

// ---------------------------------------------------------------------- list and runs
// Index-ordered place of every tile's run of segment s (an exclusive scan of the run sizes
// over its tiles, four per thread), and the segment's candidate chunks appended to the call's
// list of active chunks.  Contains barriers.
__device__ void seg_runs(const DevPlan& P, int s, uint32_t c, uint32_t* s_tmp, uint32_t* s_act) {
  // four tiles per thread and step (16 bytes a lane), four steps' loads issued together
  constexpr int kQ = 4, kSteps = 4;
  const int64_t t0 = P.tile_base[s], t1 = P.tile_base[s + 1];
  uint32_t carry = 0;
  for (int64_t tr = t0; tr < t1; tr += (int64_t)kThreads * kQ * kSteps) {
    uint32_t n[kSteps][kQ];
#pragma unroll
    for (int st = 0; st < kSteps; ++st) {
      const int64_t tq = tr + (int64_t)st * kThreads * kQ + (int64_t)threadIdx.x * kQ;
#pragma unroll
      for (int q = 0; q < kQ; ++q) n[st][q] = tq + q < t1 ? P.run_cnt[tq + q] : 0u;
    }
#pragma unroll
    for (int st = 0; st < kSteps; ++st) {
      const int64_t tq = tr + (int64_t)st * kThreads * kQ + (int64_t)threadIdx.x * kQ;
      if (tr + (int64_t)st * kThreads * kQ >= t1) break;   // uniform
      uint32_t tot;
      uint32_t run = carry + block_excl_scan<kThreads>(n[st][0] + n[st][1] + n[st][2] + n[st][3],
                                                       s_tmp, &tot);
#pragma unroll
      for (int q = 0; q < kQ; ++q) {
        if (tq + q < t1) P.run_dst[tq + q] = run;
        run += n[st][q];
      }
      carry += tot;
    }
  }
  const uint32_t nch = (c + kChunk - 1) / kChunk;
  if (threadIdx.x == 0) {
    if (carry != c) atomicOr(P.err, 8u);
    *s_act = atomicAdd(P.act_count, nch);
  }
  __syncthreads();
  for (uint32_t i = threadIdx.x; i < nch; i += kThreads)
    P.act_chunk[*s_act + i] = (uint32_t)(P.chunk_base[s] + i);
}

// ------------------------------------------------------------------------------- fallback
// The tiles of the pending segments for which pick(s) holds, in list order, dealt to the w of
// G workgroups in turn (picked tile j goes to workgroup j mod G).  The list is the call's
// pending list, or with kFromPlan the plan's segments in ascending order for which
// seg_pending holds (for a workgroup that runs beside the list's own kernel).  For each picked
// segment that has tiles here, seg_fn(s, owner) runs first (owner: this workgroup has the
// segment's first tile, so exactly one workgroup is the owner), then tile_fn(s, t) for each of
// its tiles here.  With no pending segment the function returns at once.  The picks, the
// segment loop and the tile loop are uniform over the workgroup, so both functions may
// contain barriers.
template <bool kFromPlan = false, typename Pick, typename SegFn, typename TileFn>
__device__ void for_pending_tiles(const DevPlan& P, uint32_t w, uint32_t G, Pick pick,
                                  SegFn seg_fn, TileFn tile_fn) {
  __shared__ uint32_t s_seg[kThreads];
  __shared__ uint32_t s_first[kThreads];
  __shared__ uint32_t s_tmp[kWaves];
  const uint32_t np = kFromPlan ? (uint32_t)P.n_seg : *P.pend_count;
  if (np == 0) return;   // uniform
  uint64_t rot = 0;   // picked tiles of the segments before this chunk of the list
  for (uint32_t c0 = 0; c0 < np; c0 += kThreads) {
    const uint32_t i = c0 + threadIdx.x;
    const int s = i < np ? (kFromPlan ? (int)i : (int)P.pend_list[i]) : -1;
    const bool p = s >= 0 && (!kFromPlan || seg_pending(P, s)) && pick(s);
    const uint32_t nt = p ? (uint32_t)(P.tile_base[s + 1] - P.tile_base[s]) : 0u;
    uint32_t m, tt;
    const uint32_t at = block_excl_scan<kThreads>(p ? 1u : 0u, s_tmp, &m);
    const uint32_t toff = block_excl_scan<kThreads>(nt, s_tmp, &tt);
    if (p) {
      s_seg[at] = (uint32_t)s;
      s_first[at] = (uint32_t)((w + G - (uint32_t)((rot + toff) % G)) % G);
    }
    __syncthreads();
    for (uint32_t q = 0; q < m; ++q) {
      const int si = (int)s_seg[q];
      const int64_t j0 = s_first[q];
      const int64_t t0 = P.tile_base[si], nts = P.tile_base[si + 1] - t0;
      if (j0 >= nts) continue;   // uniform: none of this segment's tiles is here
      seg_fn(si, j0 == 0);
      for (int64_t j = j0; j < nts; j += G) tile_fn(si, t0 + j);
    }
    rot += tt;
    __syncthreads();   // s_seg and s_first are rewritten for the next chunk
  }
}

// First-digit histogram of e over the pending segments, by workgroup w of G (run beside the
// list kernel, so the pending segments are found from the plan's state).
__device__ void fb_hist(const DevPlan& P, const float* __restrict__ e, uint32_t w, uint32_t G) {
  __shared__ uint32_t h[kHistBins];
  for_pending_tiles<true>(
      P, w, G, [&](int) { return true; }, [&](int, bool) {},
      [&](int s, int64_t t) { hist_tile(P, e, s, t, 0u, 0, h); });
}

// Per pending segment: the first digit of the k-th largest key.  If the keys at or above that
// bucket's floor fit the capacity, they are re-captured (kModeRecap, runs rewritten for every
// tile); otherwise the segment takes the radix select over all its elements (kModeFull) and
// its second digit is histogrammed here.  The owner workgroup records the decision.
__global__ __launch_bounds__(kThreads) void k_fb_capture(DevPlan P, const float* __restrict__ e) {
  __shared__ uint32_t h[kHistBins];
  __shared__ uint32_t s_tmp[kWaves], s_out[3], s_w[kWaves], s_base;
  uint32_t d0 = 0, kk = 0;
  bool ok = false, fits = false;
  for_pending_tiles(
      P, blockIdx.x, gridDim.x, [&](int) { return true; },
      [&](int s, bool owner) {
        const uint32_t k = call_k(P, s);
        uint32_t above, bin;
        ok = find_digit(seg_hist(P, s, 0), k, s_tmp, s_out, &d0, &above, &bin);
        fits = ok && !(P.flags & kFlagForceFull) && above + bin <= P.cand_cap[s];
        kk = ok ? k - above : 0u;
        if (owner && threadIdx.x == 0) {
          if (!ok) atomicOr(P.err, 1u);
          P.mode[s] = fits ? kModeRecap : kModeFull;
          P.thr_lo[s] = d0 << 20;
          P.pfx1[s] = d0 << 20;
          P.kk1[s] = kk;
        }
      },
      [&](int s, int64_t t) {
        if (!ok) return;   // uniform
        if (fits) {
          int64_t start;
          int len;
          tile_range(P, s, t, &start, &len);
          f4 x[kSlots];
          key_tile(P, e, start, len, x);
          capture_tile(P, s, t, start, len, x, d0 << 20, &P.recap_cnt[s], s_w, &s_base);
          __syncthreads();
        } else {
          hist_tile(P, e, s, t, d0 << 20, 1, h);
        }
      });
}

// Re-captured segments: their runs placed and chunks listed (one workgroup per segment, in
// list order); full path: the second digit, then the histogram of the last 9 bits.
__global__ __launch_bounds__(kThreads) void k_fb_hist2(DevPlan P, const float* __restrict__ e) {
  __shared__ uint32_t h[kHistBins];
  __shared__ uint32_t s_tmp[kWaves], s_out[3], s_act;
  const uint32_t np = *P.pend_count;
  if (np == 0) return;   // uniform
  for (uint32_t i = blockIdx.x; i < np; i += gridDim.x) {
    const int s = (int)P.pend_list[i];
    if (P.mode[s] != kModeRecap) continue;   // uniform
    const uint32_t c = P.recap_cnt[s];
    if (threadIdx.x == 0) P.sel_cnt[s] = c;
    seg_runs(P, s, c, s_tmp, &s_act);
    __syncthreads();
  }
  uint32_t pfx = 0;
  bool ok = false;
  for_pending_tiles(
      P, blockIdx.x, gridDim.x, [&](int s) { return P.mode[s] == kModeFull; },
      [&](int s, bool owner) {
        uint32_t d, above, bin;
        const uint32_t kk = P.kk1[s];
        ok = find_digit(seg_hist(P, s, 1), kk, s_tmp, s_out, &d, &above, &bin);
        pfx = P.pfx1[s] | (d << 9);
        if (owner && threadIdx.x == 0) {
          if (!ok) atomicOr(P.err, 1u);
          P.pfx2[s] = pfx;
          P.kk2[s] = ok ? kk - above : 0u;
        }
      },
      [&](int s, int64_t t) {
        if (ok) hist_tile(P, e, s, t, pfx, 2, h);
      });
}

// Keys above and equal to kth in one tile-shaped block (block sums).  Contains barriers.
__device__ __forceinline__ void count_block(const f4 (&x)[kSlots], int len, uint32_t kth,
                                            uint32_t* s_tmp, uint32_t* gt_out,
                                            uint32_t* eq_out) {
  const int pb = slot_base();
  uint32_t gt = 0, eq = 0;
#pragma unroll
  for (int v = 0; v < kSlots; ++v)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t key = mag_key(x[v][c]);
      const bool ok = pb + v * 256 + c < len;
      gt += (ok && key > kth) ? 1u : 0u;
      eq += (ok && key == kth) ? 1u : 0u;
    }
  *gt_out = block_sum<kThreads>(gt, s_tmp);
  *eq_out = block_sum<kThreads>(eq, s_tmp);
}

// Full path: the last digit gives the k-th key and the ties to take; then the keys above and
// at it per tile, and each tile's largest key (the int8 scale).  The owner lists the segment.
// (Its registers would halve the scatter's occupancy were it run in that launch.)
__global__ __launch_bounds__(kThreads) void k_fb_count(DevPlan P, const float* __restrict__ e) {
  __shared__ uint32_t s_tmp[kWaves], s_out[3];
  uint32_t kth = 0;
  bool ok = false;
  for_pending_tiles(
      P, blockIdx.x, gridDim.x, [&](int s) { return P.mode[s] == kModeFull; },
      [&](int s, bool owner) {
        uint32_t d, above, bin;
        const uint32_t kk = P.kk2[s];
        ok = find_digit(seg_hist(P, s, 2), kk, s_tmp, s_out, &d, &above, &bin);
        kth = P.pfx2[s] | d;
        if (owner && threadIdx.x == 0) {
          if (!ok) atomicOr(P.err, 1u);
          P.kth[s] = kth;
          P.ties[s] = ok ? kk - above : 0u;
          P.full_list[atomicAdd(P.full_count, 1u)] = (uint32_t)s;
        }
      },
      [&](int s, int64_t t) {
        if (!ok) return;   // uniform
        int64_t start;
        int len;
        tile_range(P, s, t, &start, &len);
        f4 x[kSlots];
        key_tile(P, e, start, len, x);
        uint32_t gt, eq;
        count_block(x, len, kth, s_tmp, &gt, &eq);
        uint32_t mx = 0;
        const int pb = slot_base();
#pragma unroll
        for (int v = 0; v < kSlots; ++v)
#pragma unroll
          for (int c = 0; c < 4; ++c)
            if (pb + v * 256 + c < len) mx = max(mx, mag_key(x[v][c]));
        mx = block_max<kThreads>(mx, s_tmp);
        if (threadIdx.x == 0) {
          P.tile_gt[t] = gt;
          P.tile_eq[t] = eq;
          P.tile_max[t] = mx;
        }
      });
}

// ---------------------------------------------------------------------------- cold start
// A plan's first call has no k-th key to start from.  Rather than capture nothing and
// re-capture every large segment from two extra passes over it, the call first forms acc on
// about 64 evenly spaced tiles of each such segment (exactly as the streaming pass will, but
// without storing it), histograms the first key digit, and sets the capture threshold
// GC_SAMPLE_MARGIN digits below the sample's estimate of the k-th key.  A wrong estimate only
// costs the usual re-capture: the candidates are checked for completeness as on every call.
template <bool kMomentum>
__global__ __launch_bounds__(kThreads) void k_sample_hist(DevPlan P, const float* __restrict__ g,
                                                         const float* __restrict__ e,
                                                         const float* __restrict__ u, float m) {
  __shared__ uint32_t h[kHistBins];
  const int64_t t = P.sample_tile[blockIdx.x];
  const int4 desc = P.tile_desc[t];
  const int64_t start = (int64_t)(((uint64_t)(uint32_t)desc.y << 32) | (uint32_t)desc.x);
  const int len = desc.z, s = desc.w;
  const float gf = grad_scale(P, s);
  for (int i = threadIdx.x; i < kHistBins; i += kThreads) h[i] = 0;
  f4 gv[kSlots], acc[kSlots], uv[kSlots];
  load_tile(g + start, len, gv);
  load_tile(e + start, len, acc);
  if (kMomentum) load_tile(u + start, len, uv);
  __syncthreads();
  const int pb = slot_base();
#pragma unroll
  for (int v = 0; v < kSlots; ++v) {
    f4 x = gv[v] * gf;
    if (kMomentum) {
      const f4 mu = m * uv[v];
      x = mu + x;
    }
    acc[v] = acc[v] + x;
#pragma unroll
    for (int c = 0; c < 4; ++c)
      if (pb + v * 256 + c < len) atomicAdd(&h[mag_key(acc[v][c]) >> 20], 1u);
  }
  __syncthreads();
  hist_flush(h, seg_hist(P, s, 0));
}

// Per sampled segment still without an estimate: the first-digit bucket d that holds the
// sample's ceil(k * sample / n)-th largest key; the threshold is the floor of bucket
// d - GC_SAMPLE_MARGIN.  The sample's histogram is cleared afterwards (the fallback kernels of
// the same call may need the segment's histogram).
__global__ __launch_bounds__(kThreads) void k_sample_decide(DevPlan P) {
  __shared__ uint32_t s_tmp[kWaves];
  __shared__ uint32_t s_out[3];
  const int s = blockIdx.x;
  const int64_t ns = P.sample_elems[s];
  if (ns == 0) return;
  uint32_t* h = seg_hist(P, s, 0);
  if (P.thr[s] == kNoCapture) {
    const int64_t n = P.seg_off[s + 1] - P.seg_off[s];
    const int64_t k = P.k[s];
    const uint32_t kk = (uint32_t)max((int64_t)1, (k * ns + n - 1) / n);
    uint32_t d, above, bin;
    const bool ok = find_digit(h, kk, s_tmp, s_out, &d, &above, &bin);
    if (threadIdx.x == 0 && ok)
      P.thr[s] = d > (uint32_t)GC_SAMPLE_MARGIN ? (d - (uint32_t)GC_SAMPLE_MARGIN) << 20 : 0u;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < kHistBins; i += kThreads) h[i] = 0;
}

// ------------------------------------------------------------------------------ emission
// Ordered compaction of one tile-shaped block: keep key > kth, and key == kth while the tie
// rank (eq_base + rank among the block's ties) stays below r.  slot_idx(v) gives the
// segment-local indices of this lane's slot v (loaded only for slots that keep something).
// A block whose ties are all kept or all dropped skips the tie ranking.
struct EmitOut {              // where kept entries go
  float* e;                  // residual: +0 at kept positions (or the quantisation error)
  float* u;                  // velocity to zero at kept positions, or null
  float* vals;               // kept values, or null (fused int8 call without values)
  int32_t* idx;
  int8_t* codes;             // fused int8: codes, or null
  const float* scales;       // fused int8: per-segment scales (written by the select)
  float scale;
  uint32_t seed_lo, seed_hi, step_lo;
  uint32_t* err;
  const float* vsrc;         // Random-k: kept values are read here (the tile holds keys)
  const float* rk_scale;     // Random-k without feedback: per-segment value scale, or null
  const float* vsrc_scale;   // Random-k reading g itself: the gradient scale, or null
  float vmul, gmul;
  __device__ float scales_of(int s) const { return scales[s]; }
  __device__ void set_segment(int s) {
    if (codes) scale = scales_of(s);
    if (rk_scale) vmul = rk_scale[s];
    if (vsrc_scale) gmul = vsrc_scale[s];
  }
};

template <typename SlotIdx>
__device__ __forceinline__ void emit_block(const f4 (&x)[kSlots], int len, SlotIdx slot_idx,
                                           uint32_t kth, uint32_t r, uint32_t eq_base,
                                           uint32_t eq_cnt, int64_t out_pos, int64_t out_end,
                                           int64_t s0, int32_t n_s, uint32_t* s_w,
                                           const EmitOut& o) {
  const int pb = slot_base();
  uint32_t selb[kSlots], woff[kSlots];
  const bool ties_all = (uint64_t)eq_base + eq_cnt <= r;
  const bool ties_none = eq_cnt == 0 || eq_base >= r;
  if (ties_all || ties_none) {
#pragma unroll
    for (int v = 0; v < kSlots; ++v) {
      uint32_t b = 0;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint32_t key = mag_key(x[v][c]);
        const bool ok = pb + v * 256 + c < len;
        b |= (ok && (key > kth || (ties_all && key == kth))) ? (1u << c) : 0u;
      }
      selb[v] = b;
    }
  } else {
    uint32_t eqb[kSlots];
#pragma unroll
    for (int v = 0; v < kSlots; ++v) {
      uint32_t be = 0, bg = 0;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint32_t key = mag_key(x[v][c]);
        const bool ok = pb + v * 256 + c < len;
        be |= (ok && key == kth) ? (1u << c) : 0u;
        bg |= (ok && key > kth) ? (1u << c) : 0u;
      }
      eqb[v] = be;
      selb[v] = bg;
    }
    tile_rank(eqb, woff, s_w);
#pragma unroll
    for (int v = 0; v < kSlots; ++v) {
      uint32_t q = eq_base + woff[v];
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if ((eqb[v] >> c) & 1u) {
          selb[v] |= (q < r) ? (1u << c) : 0u;
          ++q;
        }
    }
  }
  tile_rank(selb, woff, s_w);
#pragma unroll
  for (int v = 0; v < kSlots; ++v) {
    const uint32_t b = selb[v];
    if (!__ballot(b != 0)) continue;   // uniform: nothing kept in this slot of the wave
    const i4 li4 = slot_idx(v);
    int64_t q = out_pos + woff[v];
#pragma unroll
    for (int c = 0; c < 4; ++c)
      if ((b >> c) & 1u) {
        const int32_t li = li4[c];
        if (q < out_end && li >= 0 && li < n_s) {
          float val = o.vsrc ? o.vsrc[s0 + li] : x[v][c];
          if (o.vsrc_scale) val = val * o.gmul;
          if (o.rk_scale) val = val * o.vmul;
          if (o.vals) o.vals[q] = val;
          o.idx[q] = li;
          float resid = 0.0f;
          if (o.codes) {
            float deq;
            o.codes[q] = (int8_t)quant_code(val, o.scale, s0 + li, o.seed_lo, o.seed_hi,
                                            o.step_lo, &deq);
            resid = val - deq;
          }
          if (GC_NT_ZERO_E) {
            if (o.e) __builtin_nontemporal_store(resid, o.e + s0 + li);
            if (o.u) __builtin_nontemporal_store(0.0f, o.u + s0 + li);
          } else {
            if (o.e) o.e[s0 + li] = resid;
            if (o.u) o.u[s0 + li] = 0.0f;
          }
        } else {
          atomicOr(o.err, 4u);  // a rank outside the segment's output: never expected
        }
        ++q;
      }
  }
}

__device__ __forceinline__ bool has_candidates(uint32_t mode) {
  return mode == kModeCand || mode == kModeRecap;
}

// The candidate chunks of the call for chunk walker w (uniform over its workgroup), as
// f(chunk, listed): with a walker per chunk of the plan, walker w takes chunk w whatever its
// segment's state (listed false: f checks it); otherwise the call's list of the chunks of
// candidate segments (listed true), strided over the walkers.
template <typename F>
__device__ __forceinline__ void for_active_chunks(const DevPlan& P, uint32_t w, F f) {
  if ((int64_t)P.n_chunk_blocks >= P.n_chunks) {
    if ((int64_t)w < P.n_chunks) f((int64_t)w, false);
    return;
  }
  const uint32_t na = *P.act_count;
  for (uint32_t i = w; i < na; i += (uint32_t)P.n_chunk_blocks)
    f((int64_t)P.act_chunk[i], true);
}

// One chunk of a segment's candidates, in ascending index order (the select put them there).
__device__ __forceinline__ void emit_cand_chunk(const DevPlan& P, EmitOut o, int64_t ch,
                                                bool listed, uint32_t* s_w) {
  const int s = P.chunk_seg[ch];
  if (!listed && !has_candidates(P.mode[s])) return;
  const int64_t c = P.sel_cnt[s];
  const int64_t j0 = (ch - P.chunk_base[s]) * (int64_t)kChunk;
  if (j0 >= c) return;
  const int len = (int)min((int64_t)kChunk, c - j0);
  const int64_t base = P.cand_base[s] + j0;
  f4 x[kSlots];
  load_tile(P.sort_val + base, len, x);
  const int32_t* si = P.sort_idx + base;
  const int pb = slot_base();
  auto slot_idx = [&](int v) {
    i4 r;
    if (len == kTile) {
      r = reinterpret_cast<const i4*>(si)[(pb + v * 256) >> 2];
    } else {
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) r[cc] = pb + v * 256 + cc < len ? si[pb + v * 256 + cc] : 0;
    }
    return r;
  };
  o.set_segment(s);
  emit_block(x, len, slot_idx, P.kth[s], P.ties[s], P.chunk_eq_base[ch], P.chunk_eq[ch],
             P.out_off[s] + P.chunk_sel_base[ch], P.out_off[s + 1], P.seg_off[s],
             (int32_t)(P.seg_off[s + 1] - P.seg_off[s]), s_w, o);
}

// Ordered emission of one tile of a segment selected over its elements (the full path, or a
// small segment in the select kernel): the tile's keys come from e (or the Random-k keys).
__device__ __forceinline__ void emit_seg_tile(const DevPlan& P, const EmitOut& o, int s,
                                              int64_t t, uint32_t kth, uint32_t r,
                                              uint32_t eq_base, uint32_t eq_cnt,
                                              uint32_t sel_base, const f4 (&x)[kSlots],
                                              uint32_t* s_w) {
  int64_t start;
  int len;
  const int64_t s0 = P.seg_off[s];
  const int64_t st = s0 + (t - P.tile_base[s]) * (int64_t)kTile;
  const int64_t rem = P.seg_off[s + 1] - st;
  start = st;
  len = rem < kTile ? (int)rem : kTile;
  const int32_t lb = (int32_t)(start - s0) + slot_base();
  auto slot_idx = [&](int v) {
    const int32_t b0 = lb + v * 256;
    return i4{b0, b0 + 1, b0 + 2, b0 + 3};
  };
  emit_block(x, len, slot_idx, kth, r, eq_base, eq_cnt, P.out_off[s] + sel_base,
             P.out_off[s + 1], s0, (int32_t)(P.seg_off[s + 1] - s0), s_w, o);
}

__device__ __forceinline__ void emit_full_tiles(const DevPlan& P, EmitOut o, int fb, int nfb,
                                                uint32_t* s_w) {
  const uint32_t nf = *P.full_count;
  for (uint32_t li = 0; li < nf; ++li) {
    const int s = (int)P.full_list[li];
    const uint32_t kth = P.kth[s], r = P.ties[s];
    o.set_segment(s);
    for (int64_t t = P.tile_base[s] + fb; t < P.tile_base[s + 1]; t += nfb) {
      int64_t start;
      int len;
      const int64_t st = P.seg_off[s] + (t - P.tile_base[s]) * (int64_t)kTile;
      const int64_t rem = P.seg_off[s + 1] - st;
      start = st;
      len = rem < kTile ? (int)rem : kTile;
      f4 x[kSlots];
      key_tile(P, o.e, start, len, x);
      emit_seg_tile(P, o, s, t, kth, r, P.tile_eq_base[t], P.tile_eq[t], P.tile_sel_base[t], x,
                    s_w);
    }
  }
}

// ------------------------------------------------------------------------------- select
// The keys in [lo, hi] hold the k-th largest key of the segment as their kk-th largest; cnt
// of them (when known).
struct KeyRange {
  uint32_t lo, hi, kk, cnt;
};

// Histogram bins of 2^sh keys from lo.  With `window` (magnitudes above a capture threshold,
// densest just above it) the bins span at most 2^24 keys (two binades) and the top bin also
// takes every key above them; otherwise they span the whole range.
__device__ __forceinline__ int range_shift(uint32_t lo, uint32_t hi, bool window) {
  uint64_t w = (uint64_t)hi - lo + 1;
  if (window && w > ((uint64_t)1 << 24)) w = (uint64_t)1 << 24;
  int sh = 0;
  while (((w - 1) >> sh) >= (uint64_t)kHistBins) ++sh;
  return sh;
}

__device__ __forceinline__ uint32_t range_bin(uint32_t key, uint32_t lo, int sh) {
  return min((key - lo) >> sh, (uint32_t)(kHistBins - 1));
}

// Narrow r to the bin that holds its kk-th largest key, from this thread's share of the
// histogram's bins.  Contains barriers.
__device__ __forceinline__ bool range_step_in(const Bins& b, KeyRange& r, int sh, uint32_t* s_tmp,
                              uint32_t* s_out) {
  uint32_t d, above, bin;
  if (!find_digit_in(b, r.kk, s_tmp, s_out, &d, &above, &bin)) return false;
  const uint64_t nlo = (uint64_t)r.lo + ((uint64_t)d << sh);
  const uint64_t top = nlo + ((uint64_t)1 << sh) - 1;
  r.hi = (d == (uint32_t)(kHistBins - 1) || top > r.hi) ? r.hi : (uint32_t)top;
  r.lo = (uint32_t)nlo;
  r.kk -= above;
  r.cnt = bin;
  return true;
}

// range_step_in over the histogram at h (kClear: h zeroed for the next pass).  Contains
// barriers.
template <bool kClear = false>
__device__ bool range_step(uint32_t* h, KeyRange& r, int sh, uint32_t* s_tmp, uint32_t* s_out) {
  const Bins b = load_bins(h);
  if (kClear) {
#pragma unroll
    for (int j = 0; j < kHistBins / kThreads; ++j)
      h[kHistBins - 1 - (threadIdx.x * (kHistBins / kThreads) + j)] = 0;
  }
  return range_step_in(b, r, sh, s_tmp, s_out);
}

__device__ __forceinline__ void lds_clear_hist(uint32_t* h) {
  for (int i = threadIdx.x; i < kHistBins; i += kThreads) h[i] = 0;
  __syncthreads();
}

// Narrow r with histogram passes over a key source (each(f) calls f(key, position) for every
// key, each thread a share) until it holds one key value or at most cap keys.  The first
// pass may use the window (see range_shift).  h (LDS) is zero on entry and on a true return.
// Contains barriers.
template <typename Each>
__device__ bool narrow_range(Each each, KeyRange& r, bool window, uint32_t* h, uint32_t* s_tmp,
                             uint32_t* s_out, uint32_t cap = kListCap) {
  bool first = true;
  for (int it = 0; r.hi > r.lo && r.cnt > cap; ++it) {
    if (it == 8) return false;
    const int sh = range_shift(r.lo, r.hi, window && first);
    const uint32_t lo = r.lo, hi = r.hi;
    each([&](uint32_t key, uint32_t) {
      if (key >= lo && key <= hi) atomicAdd(&h[range_bin(key, lo, sh)], 1u);
    });
    __syncthreads();
    if (!range_step<true>(h, r, sh, s_tmp, s_out)) return false;
    first = false;
  }
  return true;
}

// The exact k-th key inside r from the n keys of the LDS list (every key of the source that
// lies in r).  On return r.lo == r.hi is the key and r.kk the ties to take.  h (LDS) is zero on
// entry and on a true return.
__device__ bool list_select(const uint32_t* lkey, uint32_t n, KeyRange& r, uint32_t* h,
                            uint32_t* s_tmp, uint32_t* s_out) {
  for (int it = 0; r.hi > r.lo; ++it) {
    if (it == 4) return false;
    const int sh = range_shift(r.lo, r.hi, false);
    for (uint32_t i = threadIdx.x; i < n; i += kThreads) {
      const uint32_t key = lkey[i];
      if (key >= r.lo && key <= r.hi) atomicAdd(&h[range_bin(key, r.lo, sh)], 1u);
    }
    __syncthreads();
    if (!range_step<true>(h, r, sh, s_tmp, s_out)) return false;
  }
  return true;
}

// LDS of the finish kernel.
struct alignas(16) SelLds {
  uint32_t h[kHistBins];
  uint32_t lkey[kListCap];
  uint32_t lch[kListCap];        // a near list held whole: each entry's output chunk
  uint32_t cgt[kFinishChunks];   // per output chunk of a window: near keys above kth
  uint32_t ceq[kFinishChunks];   // and at kth
  uint32_t tmp[kWaves];
  uint32_t out[3];
  uint32_t w[kWaves];
  uint32_t n_list;
};

// The segment's key range after the candidates' windowed histogram (k_scatter): the bin that
// holds its k-th key.  Histogram bins of 2^sh keys from the capture floor lo (window: at most
// two binades above it, the top bin taking everything above).  Contains barriers.
__device__ __forceinline__ bool cand_range_in(const DevPlan& P, int s, uint32_t k,
                                              const Bins& b, KeyRange* r, uint32_t* s_tmp,
                                              uint32_t* s_out) {
  const uint32_t lo = P.thr_lo[s];
  const bool window = P.keys == kKeysMagnitude && lo > 0;
  const int sh = range_shift(lo, 0x7FFFFFFFu, window);
  *r = KeyRange{lo, 0x7FFFFFFFu, k, P.sel_cnt[s]};
  return range_step_in(b, *r, sh, s_tmp, s_out);
}

__device__ __forceinline__ bool cand_range(const DevPlan& P, int s, uint32_t k, KeyRange* r,
                                           uint32_t* s_tmp, uint32_t* s_out) {
  return cand_range_in(P, s, k, load_bins(seg_hist(P, s, 1)), r, s_tmp, s_out);
}

// Most keys that rank_select takes (it compares each key with every other).
constexpr uint32_t kRankMax = 256;

// The kk-th largest of the n <= kRankMax keys of an LDS list (16-byte aligned), by counting:
// q threads per key (q a power of two, q * n <= kThreads), each comparing it with its own
// contiguous part of the list, so that its count of keys above it and at it is exact.  On
// return r is that one key and r.kk the ties to take.  s_out: LDS uint32_t[3].  Contains
// barriers.
__device__ bool rank_select(const uint32_t* lkey, uint32_t n, KeyRange& r, uint32_t* s_out) {
  uint32_t q = 1;
  while (q < 64 && q * 2 * n <= (uint32_t)kThreads) q *= 2;
  const uint32_t j = threadIdx.x / q, part = threadIdx.x % q, kk = r.kk;
  const uint32_t per = ((n + q - 1) / q + 3) & ~3u;   // whole 16-byte groups per part
  if (threadIdx.x == 0) s_out[2] = 0;
  __syncthreads();
  const uint32_t kj = j < n ? lkey[j] : 0u;
  uint32_t gt = 0, eq = 0;
  if (j < n) {
    const uint32_t i0 = part * per, i1 = min(n, i0 + per);
    uint32_t i = i0;
#pragma unroll 4
    for (; i + 4 <= i1; i += 4) {
      const uint4 v = *reinterpret_cast<const uint4*>(lkey + i);
      gt += (v.x > kj ? 1u : 0u) + (v.y > kj ? 1u : 0u) + (v.z > kj ? 1u : 0u) +
            (v.w > kj ? 1u : 0u);
      eq += (v.x == kj ? 1u : 0u) + (v.y == kj ? 1u : 0u) + (v.z == kj ? 1u : 0u) +
            (v.w == kj ? 1u : 0u);
    }
    for (; i < i1; ++i) {
      const uint32_t ki = lkey[i];
      gt += ki > kj ? 1u : 0u;
      eq += ki == kj ? 1u : 0u;
    }
  }
  for (uint32_t d = 1; d < q; d <<= 1) {
    gt += __shfl_xor(gt, (int)d, 64);
    eq += __shfl_xor(eq, (int)d, 64);
  }
  if (j < n && part == 0 && gt < kk && kk <= gt + eq) {   // every such thread holds the same key
    s_out[0] = kj;
    s_out[1] = kk - gt;
    s_out[2] = 1;
  }
  __syncthreads();
  const bool found = s_out[2] != 0;
  if (found) {
    r.lo = r.hi = s_out[0];
    r.kk = s_out[1];
  }
  __syncthreads();
  return found;
}

// ------------------------------------------------------------------------------ scatter
// Candidates into ascending index order (tile t's run goes to run_dst[t]), the windowed
// histogram of their keys (seg_hist slot 1) and each chunk's largest key.  One chunk of the
// call's list of active chunks; contains barriers.
__device__ void scatter_chunk(const DevPlan& P, int64_t ch, bool listed, uint32_t* h,
                              uint32_t* s_m) {
  const int s = P.chunk_seg[ch];
  if (!listed && !has_candidates(P.mode[s])) return;   // uniform
  const int64_t c = P.sel_cnt[s];
  const int64_t j0 = (ch - P.chunk_base[s]) * (int64_t)kChunk;
  if (j0 >= c) return;   // uniform: a chunk past the segment's candidates
  const uint32_t lo = P.thr_lo[s];
  const bool window = P.keys == kKeysMagnitude && lo > 0;
  const int sh = range_shift(lo, 0x7FFFFFFFu, window);
  for (int i = threadIdx.x; i < kHistBins; i += kThreads) h[i] = 0;
  const int len = (int)min((int64_t)kChunk, c - j0);
  const int64_t cb = P.cand_base[s], tb = P.tile_base[s];
  const int32_t n_s = (int32_t)(P.seg_off[s + 1] - P.seg_off[s]);
  constexpr int kPer = kChunk / kThreads;
  int32_t ix[kPer];
  float vx[kPer];
#pragma unroll
  for (int r = 0; r < kPer; ++r) {
    const int p = r * kThreads + threadIdx.x;
    ix[r] = p < len ? P.cand_idx[cb + j0 + p] : 0;
    vx[r] = p < len ? P.cand_val[cb + j0 + p] : 0.0f;
  }
  uint32_t rd[kPer], ro[kPer];
#pragma unroll
  for (int r = 0; r < kPer; ++r) {
    const int64_t t = tb + (ix[r] >= 0 && ix[r] < n_s ? ix[r] / kTile : 0);
    rd[r] = P.run_dst[t];
    ro[r] = P.run_off[t];
  }
  __syncthreads();   // h cleared
  uint32_t mx = 0, bad = 0;
#pragma unroll
  for (int r = 0; r < kPer; ++r) {
    const int p = r * kThreads + threadIdx.x;
    if (p < len) {
      const uint32_t key = mag_key(vx[r]);
      const uint32_t dst = rd[r] + ((uint32_t)(j0 + p) - ro[r]);
      if (ix[r] >= 0 && ix[r] < n_s && dst < (uint32_t)c && key >= lo) {
        P.sort_val[cb + dst] = vx[r];
        P.sort_idx[cb + dst] = ix[r];
        atomicAdd(&h[range_bin(key, lo, sh)], 1u);
        mx = max(mx, key);
      } else {
        bad = 1;
      }
    }
  }
  if (bad) atomicOr(P.err, 8u);
  mx = block_max<kThreads>(mx, s_m);
  if (threadIdx.x == 0) P.chunk_max[ch] = mx;
  hist_flush(h, seg_hist(P, s, 1));
}

__global__ __launch_bounds__(kThreads, 8) void k_scatter(DevPlan P) {
  __shared__ uint32_t h[kHistBins];
  __shared__ uint32_t s_m[kWaves];
  for_active_chunks(P, blockIdx.x, [&](int64_t ch, bool listed) {
    scatter_chunk(P, ch, listed, h, s_m);
    __syncthreads();   // the next chunk reuses h
  });
}

// ------------------------------------------------------------------------------ collect
// Per chunk of ordered candidates: the keys above the range that holds the segment's k-th
// key (chunk_gt), and the keys inside it appended to the segment's near list (key bits in the
// free unordered candidate region, ordered position beside them).  The range comes from the
// windowed histogram, derived again by each workgroup for the segments of its chunks.
__global__ __launch_bounds__(kThreads, 8) void k_collect(DevPlan P) {
  __shared__ uint32_t s_tmp[kWaves], s_out[3], s_w[kWaves], s_base;
  int cur = -1;
  KeyRange r{0u, 0u, 0u, 0u};
  bool ok = false;
  for_active_chunks(P, blockIdx.x, [&](int64_t ch, bool listed) {
    const int s = P.chunk_seg[ch];
    if (!listed && !has_candidates(P.mode[s])) return;   // uniform
    const int64_t c = P.sel_cnt[s];
    const int64_t j0 = (ch - P.chunk_base[s]) * (int64_t)kChunk;
    if (j0 >= c) return;   // uniform
    if (s != cur) {   // uniform
      ok = cand_range(P, s, call_k(P, s), &r, s_tmp, s_out);
      cur = s;
      if (!ok && threadIdx.x == 0) atomicOr(P.err, 1u);
    }
    if (!ok) return;   // uniform
    const int len = (int)min((int64_t)kChunk, c - j0);
    const int64_t cb = P.cand_base[s];
    f4 x[kSlots];
    load_tile(P.sort_val + cb + j0, len, x);
    const int pb = slot_base();
    uint32_t near[kSlots], gt = 0;
#pragma unroll
    for (int v = 0; v < kSlots; ++v) {
      uint32_t b = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t key = mag_key(x[v][q]);
        const bool in = pb + v * 256 + q < len;
        gt += (in && key > r.hi) ? 1u : 0u;
        b |= (in && key >= r.lo && key <= r.hi) ? (1u << q) : 0u;
      }
      near[v] = b;
    }
    uint32_t woff[kSlots];
    const uint32_t total = tile_rank(near, woff, s_w);
    gt = block_sum<kThreads>(gt, s_tmp);
    if (threadIdx.x == 0) {
      P.chunk_gt[ch] = gt;
      s_base = total ? atomicAdd(&P.near_cnt[s], total) : 0u;
    }
    __syncthreads();
    const uint32_t base = s_base;
    float* nk = P.cand_val + cb;
    int32_t* np = P.cand_idx + cb;
#pragma unroll
    for (int v = 0; v < kSlots; ++v) {
      uint32_t q = base + woff[v];
#pragma unroll
      for (int cc = 0; cc < 4; ++cc)
        if ((near[v] >> cc) & 1u) {
          nk[q] = x[v][cc];
          np[q] = (int32_t)(j0 + pb + v * 256 + cc);
          ++q;
        }
    }
    __syncthreads();   // s_base is rewritten for the next chunk
  });
}

// Near-list source: f(key, j) for the n entries at v (keys stored as float bits).
struct NearKeys {
  const float* v;
  uint32_t n;
  template <typename F>
  __device__ __forceinline__ void operator()(F f) const {
    for (uint32_t j = threadIdx.x; j < n; j += kThreads) f(mag_key(v[j]), j);
  }
};

// Candidate segment after k_collect: the exact k-th key and ties from its near list (in LDS
// when small enough, else narrowed first by histogram passes over it), the near keys added to
// their chunks' counts, and the per-chunk offsets of the ordered emission.  Returns the
// largest key in *mx.  Contains barriers.
__device__ void finish_cands(const DevPlan& P, int s, uint32_t k, SelLds& L, uint32_t* kth_out,
                             uint32_t* ties_out, uint32_t* mx_out) {
  // loads that do not wait on one another first: the windowed histogram, the counts, and the
  // first chunks' counts above the range and largest keys
  const Bins hb = load_bins(seg_hist(P, s, 1));
  const uint32_t c = P.sel_cnt[s], n_near = P.near_cnt[s];
  const int64_t cb = P.cand_base[s], ch0 = P.chunk_base[s];
  const uint32_t nch = (c + kChunk - 1) / kChunk;
  uint32_t gt0 = 0, mx0 = 0;
  if (threadIdx.x < nch) {
    gt0 = P.chunk_gt[ch0 + threadIdx.x];
    mx0 = P.chunk_max[ch0 + threadIdx.x];
  }
  const NearKeys near{P.cand_val + cb, n_near};
  const int32_t* npos = P.cand_idx + cb;
  // a near list that fits in LDS is read once: every entry's key and output chunk
  const bool in_lds = n_near <= (uint32_t)kListCap;
  for (int i = threadIdx.x; i < kHistBins; i += kThreads) L.h[i] = 0;
  if (threadIdx.x == 0) L.n_list = 0;
  if (in_lds) {
    for (uint32_t j = threadIdx.x; j < n_near; j += kThreads) {
      L.lkey[j] = mag_key(near.v[j]);
      L.lch[j] = (uint32_t)npos[j] / kChunk;
    }
  }
  KeyRange r;
  bool ok = cand_range_in(P, s, k, hb, &r, L.tmp, L.out);   // (its barriers order the above)
  if (ok && n_near != r.cnt) ok = false;   // the list holds exactly the bin's keys
  uint32_t bad = ok ? 0u : 1u;
  if (in_lds) {
    if (ok && r.hi > r.lo) {
      const bool found = n_near <= kRankMax
                             ? rank_select(L.lkey, n_near, r, L.out)
                             : list_select(L.lkey, n_near, r, L.h, L.tmp, L.out);
      if (!found) bad = 1;
    }
  } else {
    if (ok) ok = narrow_range(near, r, false, L.h, L.tmp, L.out);
    bad = ok ? 0u : 1u;
    if (ok && r.hi > r.lo) {
      // the keys inside r into the LDS list: one slot reservation per wave and step
      near([&](uint32_t key, uint32_t) {
        const bool in = key >= r.lo && key <= r.hi;
        const uint64_t m = __ballot(in);
        if (m == 0) return;
        const int lead = __ffsll((unsigned long long)m) - 1;
        uint32_t base = 0;
        if (lane_id() == lead) base = atomicAdd(&L.n_list, (uint32_t)__popcll(m));
        base = __shfl(base, lead, 64);
        if (in) {
          const uint32_t p = base + lanes_below(m);
          if (p < (uint32_t)kListCap) L.lkey[p] = key;
          else bad = 1;
        }
      });
      bad = block_max<kThreads>(bad, L.tmp);
      if (!bad && !list_select(L.lkey, min(L.n_list, (uint32_t)kListCap), r, L.h, L.tmp, L.out))
        bad = 1;
    }
  }
  const uint32_t kth = r.lo, ties = r.kk;
  // per output chunk: the keys above kth (k_collect's count above the range plus the near
  // keys above kth) and at kth (near keys only), counted in LDS for windows of kFinishChunks
  // chunks; then the ties before each chunk and the kept entries before it: the keys above
  // kth before it plus the first `ties` of the ties before it
  uint32_t ce = 0, cg = 0, mx = 0;
  for (uint32_t w0 = 0; w0 < nch; w0 += kFinishChunks) {
    const uint32_t wn = min(nch - w0, (uint32_t)kFinishChunks);
    for (uint32_t i = threadIdx.x; i < wn; i += kThreads) {
      L.cgt[i] = 0;
      L.ceq[i] = 0;
    }
    __syncthreads();
    auto count = [&](uint32_t key, uint32_t ch) {
      if (ch < w0 || ch >= w0 + wn) return;
      if (key > kth) atomicAdd(&L.cgt[ch - w0], 1u);
      else if (key == kth) atomicAdd(&L.ceq[ch - w0], 1u);
    };
    if (!bad && in_lds) {
      for (uint32_t j = threadIdx.x; j < n_near; j += kThreads) count(L.lkey[j], L.lch[j]);
    } else if (!bad) {
      near([&](uint32_t key, uint32_t j) { count(key, (uint32_t)npos[j] / kChunk); });
    }
    __syncthreads();
    for (uint32_t i0 = 0; i0 < wn; i0 += kThreads) {
      const uint32_t i = i0 + threadIdx.x;
      const bool in = i < wn;
      const int64_t ch = ch0 + w0 + i;
      const bool first = w0 + i0 == 0;   // uniform: the chunks loaded up front
      uint32_t eq = 0, gt = 0;
      if (in) {
        eq = L.ceq[i];
        gt = (first ? gt0 : P.chunk_gt[ch]) + L.cgt[i];
        mx = max(mx, first ? mx0 : P.chunk_max[ch]);
      }
      uint32_t eqb, gtb, te, tg;
      block_excl_scan2<kThreads>(eq, gt, L.tmp, L.w, &eqb, &gtb, &te, &tg);
      eqb += ce;
      gtb += cg;
      if (in) {
        P.chunk_eq[ch] = eq;
        P.chunk_eq_base[ch] = eqb;
        P.chunk_sel_base[ch] = gtb + min(eqb, ties);
      }
      ce += te;
      cg += tg;
    }
    __syncthreads();   // the counters are cleared for the next window
  }
  if (threadIdx.x == 0) {
    if (bad) atomicOr(P.err, 16u);
    if (cg + min(ce, ties) != k) atomicOr(P.err, 2u);
  }
  *kth_out = kth;
  *ties_out = ties;
  *mx_out = block_max<kThreads>(mx, L.tmp);
}

// Full path: the per-tile counts of the keys above and at kth (fb_count) scanned in tile order
// into the tiles' ordered-emission offsets; returns the largest key.  Contains barriers.
__device__ uint32_t select_full_scan(const DevPlan& P, int s, uint32_t k, uint32_t ties,
                                     SelLds& L) {
  const int64_t t0 = P.tile_base[s], t1 = P.tile_base[s + 1];
  uint32_t ce = 0, cg = 0, mx = 0;
  for (int64_t tb = t0; tb < t1; tb += kThreads) {
    const int64_t t = tb + threadIdx.x;
    const bool in = t < t1;
    const uint32_t gt = in ? P.tile_gt[t] : 0u, eq = in ? P.tile_eq[t] : 0u;
    if (in) mx = max(mx, P.tile_max[t]);
    uint32_t eqb, gtb, te, tg;
    block_excl_scan2<kThreads>(eq, gt, L.tmp, L.w, &eqb, &gtb, &te, &tg);
    eqb += ce;
    gtb += cg;
    if (in) {   // kept before the tile: its keys above kth and the first `ties` of its ties
      P.tile_eq_base[t] = eqb;
      P.tile_sel_base[t] = gtb + min(eqb, ties);
    }
    ce += te;
    cg += tg;
  }
  if (threadIdx.x == 0 && cg + min(ce, ties) != k) atomicOr(P.err, 2u);
  return block_max<kThreads>(mx, L.tmp);
}

// Sums over a block of N values per thread at once (one pair of barriers); scratch: LDS of
// N * kWaves words.
template <int N>
__device__ __forceinline__ void block_sums(uint32_t (&v)[N], uint32_t* scratch) {
#pragma unroll
  for (int i = 0; i < N; ++i)
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) v[i] += __shfl_xor(v[i], d, 64);
  if (lane_id() == 0) {
#pragma unroll
    for (int i = 0; i < N; ++i) scratch[i * kWaves + wave_id()] = v[i];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < N; ++i) {
    uint32_t t = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) t += scratch[i * kWaves + w];
    v[i] = t;
  }
  __syncthreads();
}

// LDS of a small segment's select (in the emission kernel).
// The exact k-th key (and the ties to take) of a key source whose k-th key lies in [lo, hi]:
// a histogram of the keys in [lo, hi] (bins of 2^sh keys from lo; with `window`, magnitudes
// above a capture floor, bins of 2^13 keys over two binades, the top bin open) picks the bin
// that holds the k-th key; the bin's keys are narrowed by further histogram passes while more
// than L.cap, then gathered into the LDS list L.lkey and ranked there (by counting for at
// most kRankMax keys).  each(f) calls f(key) for every key of the source, each thread a
// share; *mx (if given): this thread's largest key.  False when [lo, hi] holds fewer than k
// keys (or on a list past its capacity).  L.h is zero on entry and on a true return.
// Contains barriers.
struct NearLds {
  uint32_t* h;        // kHistBins
  uint32_t* tmp;      // kWaves
  uint32_t* out;      // 3
  uint32_t* n_list;
  uint32_t* lkey;     // cap keys, 16-byte aligned
  uint32_t cap;
};

template <typename Each>
__device__ __forceinline__ bool near_select(Each each, uint32_t lo, uint32_t hi, bool window,
                                            uint32_t k, const NearLds& L, uint32_t* kth,
                                            uint32_t* ties, uint32_t* mx = nullptr) {
  const int sh = range_shift(lo, hi, window);
  uint32_t m = 0;
  each([&](uint32_t key) {
    m = max(m, key);
    if (key >= lo && key <= hi) atomicAdd(&L.h[range_bin(key, lo, sh)], 1u);
  });
  if (mx) *mx = m;
  if (threadIdx.x == 0) *L.n_list = 0;
  __syncthreads();
  KeyRange r{lo, hi, k, 0u};
  if (!range_step<true>(L.h, r, sh, L.tmp, L.out)) return false;
  if (r.hi > r.lo) {
    auto each_at = [&](auto f) { each([&](uint32_t key) { f(key, 0u); }); };
    if (!narrow_range(each_at, r, false, L.h, L.tmp, L.out, L.cap)) return false;
  }
  if (r.hi > r.lo) {   // uniform
    // the keys inside r into the list: one slot reservation per wave and step
    uint32_t bad = 0;
    each([&](uint32_t key) {
      const bool in = key >= r.lo && key <= r.hi;
      const uint64_t b = __ballot(in);
      if (b == 0) return;
      const int lead = __ffsll((unsigned long long)b) - 1;
      uint32_t base = 0;
      if (lane_id() == lead) base = atomicAdd(L.n_list, (uint32_t)__popcll(b));
      base = __shfl(base, lead, 64);
      if (in) {
        const uint32_t p = base + lanes_below(b);
        if (p < L.cap) L.lkey[p] = key;
        else bad = 1;
      }
    });
    if (block_max<kThreads>(bad, L.tmp)) return false;   // (its barriers order the list)
    const uint32_t n = *L.n_list;
    if (!(n <= kRankMax ? rank_select(L.lkey, n, r, L.out)
                        : list_select(L.lkey, n, r, L.h, L.tmp, L.out)))
      return false;
  }
  *kth = r.lo;
  *ties = r.kk;
  return true;
}

struct alignas(16) SmallLds {
  uint32_t h[kHistBins];
  uint32_t lkey[kRankMax];   // the select's near list
  uint32_t sums[kSmallTiles * kWaves];
  uint32_t tmp[kWaves];
  uint32_t out[3];
  uint32_t w[kWaves];
  uint32_t n_list;
};

// Small segment (at most kSmallTiles tiles): selected whole from its residual (or Random-k
// keys), every key loaded once into registers.  The exact k-th key by near_select over the
// eight binades below the segment's largest key (2048 bins of 2^15 keys: a radix digit of 11
// bits would pile the bulk of the keys onto a few bins, serialising the LDS atomics), or, when
// fewer than k keys lie there, by a radix select over the registers (digits of 11, 11 and 9
// bits, as the full path); then the segment emitted in index order, tile by tile.  Returns
// kth, ties and the largest key.  Contains barriers.
__device__ __forceinline__ void select_small(const DevPlan& P, const float* e,
                                             const EmitOut& o, int s, uint32_t k, SmallLds& L,
                                             uint32_t* kth_out, uint32_t* ties_out,
                                             uint32_t* mx_out) {
  static_assert(kTile < 65536, "a tile's counts are packed in 16 bits");
  const int64_t t0 = P.tile_base[s];
  const int nt = (int)(P.tile_base[s + 1] - t0);
  const int pb = slot_base();
  f4 x[kSmallTiles][kSlots];
  int len[kSmallTiles];
#pragma unroll
  for (int j = 0; j < kSmallTiles; ++j) {
    len[j] = 0;
    if (j < nt) {
      int64_t start;
      tile_range(P, s, t0 + j, &start, &len[j]);
      key_tile(P, e, start, len[j], x[j]);
    } else {
#pragma unroll
      for (int v = 0; v < kSlots; ++v) x[j][v] = f4{0.0f, 0.0f, 0.0f, 0.0f};
    }
  }
  for (int i = threadIdx.x; i < kHistBins; i += kThreads) L.h[i] = 0;
  auto keys = [&](auto f) {
#pragma unroll
    for (int j = 0; j < kSmallTiles; ++j)
#pragma unroll
      for (int v = 0; v < kSlots; ++v)
#pragma unroll
        for (int c = 0; c < 4; ++c)
          if (pb + v * 256 + c < len[j]) f(mag_key(x[j][v][c]));
  };
  uint32_t mx = 0;
  keys([&](uint32_t key) { mx = max(mx, key); });
  mx = block_max<kThreads>(mx, L.tmp);   // (its barriers order the histogram's clearing)
  constexpr uint32_t kSpan = (1u << 26) - 1;   // eight binades of keys
  const NearLds nl{L.h, L.tmp, L.out, &L.n_list, L.lkey, kRankMax};
  uint32_t kth = 0, ties = 0;
  bool ok = k > 0 && near_select(keys, mx > kSpan ? mx - kSpan : 0u, mx, false, k, nl, &kth,
                                 &ties);
  if (!ok) {   // uniform: the k-th key lies further down
    lds_clear_hist(L.h);
    uint32_t prefix = 0, kk = k;
    ok = true;
    for (int pass = 0; pass < 3; ++pass) {
#pragma unroll
      for (int j = 0; j < kSmallTiles; ++j) hist_add(L.h, x[j], len[j], prefix, pass);
      __syncthreads();
      uint32_t d, above, bin;
      if (!find_digit<true>(L.h, kk, L.tmp, L.out, &d, &above, &bin)) {   // uniform
        ok = false;
        break;
      }
      prefix |= d << digit_shift(pass);
      kk -= above;
    }
    kth = prefix;
    ties = kk;
  }
  if (ok) {
    EmitOut os = o;
    if (os.codes) os.scale = __uint_as_float(mx) / 127.0f;
    if (os.rk_scale) os.vmul = os.rk_scale[s];
    if (os.vsrc_scale) os.gmul = os.vsrc_scale[s];
    // per tile: the keys above kth (low half) and at it (high half), all tiles in one reduction
    uint32_t cnt[kSmallTiles];
#pragma unroll
    for (int j = 0; j < kSmallTiles; ++j) {
      uint32_t gt = 0, eq = 0;
#pragma unroll
      for (int v = 0; v < kSlots; ++v)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const uint32_t key = mag_key(x[j][v][c]);
          const bool in = pb + v * 256 + c < len[j];
          gt += (in && key > kth) ? 1u : 0u;
          eq += (in && key == kth) ? 1u : 0u;
        }
      cnt[j] = gt | (eq << 16);
    }
    block_sums<kSmallTiles>(cnt, L.sums);
    uint32_t eqb = 0, kept = 0;
#pragma unroll
    for (int j = 0; j < kSmallTiles; ++j) {
      if (j >= nt) break;   // uniform
      const uint32_t gt = cnt[j] & 0xFFFFu, eq = cnt[j] >> 16;
      emit_seg_tile(P, os, s, t0 + j, kth, ties, eqb, eq, kept, x[j], L.w);
      kept += gt + (eqb < ties ? min(eq, ties - eqb) : 0u);
      eqb += eq;
    }
    if (threadIdx.x == 0 && kept != k) atomicOr(P.err, 2u);
  } else if (threadIdx.x == 0) {
    atomicOr(P.err, 16u);
  }
  *kth_out = kth;
  *ties_out = ties;
  *mx_out = mx;
}

// First after the streaming pass.  Workgroups [0, n_seg): one per segment, the segment's path
// this call.  k = 0: nothing (its counters cleared).  Small: selected and emitted whole by the
// emission kernel (it needs no fallback).  Candidates complete: the places of its runs, its
// chunks listed, its capture floor.  Otherwise: listed as pending for the fallback kernels.
// The rest: the first-digit histogram of the pending segments.
__global__ __launch_bounds__(kThreads) void k_list(DevPlan P, const float* __restrict__ e) {
  __shared__ uint32_t s_tmp[kWaves];
  __shared__ uint32_t s_act;
  if (blockIdx.x >= (uint32_t)P.n_seg) {   // uniform
    fb_hist(P, e, blockIdx.x - (uint32_t)P.n_seg, gridDim.x - (uint32_t)P.n_seg);
    return;
  }
  const int s = blockIdx.x;
  const uint32_t k = call_k(P, s);
  uint32_t mode = kModeCand;
  if (k == 0) mode = kModeSkip;
  else if (P.seg_flags[s] & kSegSmall) mode = kModeSmall;
  else if (seg_pending(P, s)) mode = kModePending;
  if (mode != kModeCand) {
    if (threadIdx.x == 0) {
      P.mode[s] = mode;
      if (mode == kModePending) P.pend_list[atomicAdd(P.pend_count, 1u)] = (uint32_t)s;
    }
    return;
  }
  const uint32_t c = P.cand_cnt[s];
  if (threadIdx.x == 0) {
    P.mode[s] = kModeCand;
    P.sel_cnt[s] = c;
    P.thr_lo[s] = capture_thr(P, s);
  }
  seg_runs(P, s, c, s_tmp, &s_act);
}

// Last per-segment step of a call (every thread of the workgroup): the threshold call's
// count and its unused slots padded with (+0, -1); the statistics; the next capture threshold
// (beta * |kth|, the margin beta steered by the last calls: lowered after too few candidates,
// raised after an overflow or far more than needed, kept in [0.25, GC_BETA_MAX]; segments that
// capture everything or nothing keep their setting); the per-call counters cleared.  pend: the
// capture was incomplete; c_cap: candidates the pass captured; c_sel: candidates the select
// ran over.  A small segment's kth, ties and scale are written by its select.
__device__ __forceinline__ void finalize_segment(const DevPlan& P, const EmitOut& o, int s,
                                                 uint32_t k, uint32_t mode, bool pend,
                                                 uint32_t thr_used, uint32_t c_cap,
                                                 uint32_t c_sel, uint32_t kth, uint32_t ties,
                                                 uint32_t mx) {
  if (P.codec == kCodecThreshold) {
    const int64_t a = P.out_off[s] + k, b = P.out_off[s + 1];
    for (int64_t j = a + threadIdx.x; j < b; j += kThreads) {
      o.vals[j] = 0.0f;
      o.idx[j] = -1;
    }
  }
  if (threadIdx.x != 0) return;
  if (P.out_count) P.out_count[s] = (int32_t)k;
  if (P.scales && mode != kModeSmall) P.scales[s] = k ? __uint_as_float(mx) / 127.0f : 0.0f;
  P.sel_cnt[s] = c_sel;
  if (mode != kModeSmall) {
    P.kth[s] = kth;
    P.ties[s] = ties;
  }
  const bool steer = mode != kModeSmall && k > 0 && P.thr_init[s] == kNoCapture &&
                     !(P.flags & (kFlagForceFull | kFlagNoEstimate));
  if (P.codec == kCodecTopk || P.codec == kCodecThreshold) {
    float* beta = P.codec == kCodecTopk ? P.beta : P.beta_est;
    if (steer) {
      float b = beta[s];
      if (pend) {
        if (thr_used != kNoCapture) {
          if (c_cap < k) b = fmaxf(b * 0.85f, 0.25f);                // missed
          else b = fminf(b * 1.05f, GC_BETA_MAX);                     // overflowed
        }
      } else {
        const float rho = (float)c_cap / (float)k;
        if (rho > GC_RHO_HIGH) b = fminf(b * 1.03f, GC_BETA_MAX);
        else if (rho < GC_RHO_LOW) b = fmaxf(b * 0.97f, 0.25f);
      }
      beta[s] = b;
      const uint32_t next = mag_key(b * __uint_as_float(kth));
      if (P.codec == kCodecTopk) P.thr[s] = next;
      else P.thr_est[s] = next;
    } else if (P.codec == kCodecTopk) {
      P.thr[s] = P.thr_init[s];
    }
  }
  P.cand_cnt[s] = 0;
  P.recap_cnt[s] = 0;
  if (mode != kModeSmall) P.tau_cnt[s] = 0;   // a small segment's k is read by its select later
  P.near_cnt[s] = 0;
}

// One workgroup per segment, last before the emission: the segment's exact k-th key and ties
// (candidate path: from its near list; full path: from fb_count), the offsets of its ordered
// emission, the int8 scale, the threshold call's count and padding, the call's statistics,
// the next capture threshold, and the per-call counters and histograms cleared for the next
// call.
__global__ __launch_bounds__(kThreads) void k_finish(DevPlan P, const float* __restrict__ e,
                                                    EmitOut o) {
  __shared__ SelLds L;
  const int s = blockIdx.x;
  const uint32_t k = call_k(P, s);
  const uint32_t mode = P.mode[s];
  const bool pend = mode == kModeRecap || mode == kModeFull;
  const uint32_t thr_used = capture_thr(P, s);
  const uint32_t c_cap = P.cand_cnt[s];
  uint32_t kth = 0, ties = 0, mx = 0, c_sel = 0;
  if (mode == kModeCand || mode == kModeRecap) {
    c_sel = P.sel_cnt[s];
    finish_cands(P, s, k, L, &kth, &ties, &mx);
  } else if (mode == kModeFull) {
    kth = P.kth[s];
    ties = P.ties[s];
    mx = select_full_scan(P, s, k, ties, L);
  }
  // histograms used by this call, cleared for the next one: the candidates' windowed one
  // (slot 1) and, for a pending segment, the fallback's three
  if (mode == kModeCand || pend) {
    uint32_t* h = seg_hist(P, s, pend ? 0 : 1);
    const int nb = (pend ? 3 : 1) * kHistBins;
    for (int i = threadIdx.x; i < nb; i += kThreads) h[i] = 0;
  }
  finalize_segment(P, o, s, k, mode, pend, thr_used, c_cap, c_sel, kth, ties, mx);
}

// The last kernel of a call.  Workgroups [0, n_seg): a small segment each (selected and
// emitted whole, from its residual, alongside the rest: no other kernel waits for it); then
// n_chunk_blocks over the active candidate chunks; the rest over the tiles of the segments on
// the full path.
__global__ __launch_bounds__(kThreads) void k_emit(DevPlan P, const float* __restrict__ e,
                                                  EmitOut o) {
  __shared__ SmallLds L;
  const uint32_t b = blockIdx.x;
  if (b < (uint32_t)P.n_seg) {
    const int s = (int)b;
    if (P.mode[s] != kModeSmall) return;   // uniform
    uint32_t kth, ties, mx;
    select_small(P, e, o, s, call_k(P, s), L, &kth, &ties, &mx);
    if (threadIdx.x == 0) {
      if (P.scales) P.scales[s] = __uint_as_float(mx) / 127.0f;
      P.kth[s] = kth;
      P.ties[s] = ties;
      P.tau_cnt[s] = 0;   // the threshold call's count, read above, cleared for the next call
    }
    return;
  }
  const uint32_t c0 = b - (uint32_t)P.n_seg;
  if (c0 < (uint32_t)P.n_chunk_blocks) {
    for_active_chunks(P, c0, [&](int64_t ch, bool listed) {
      emit_cand_chunk(P, o, ch, listed, L.w);
    });
  } else {
    const uint32_t f0 = c0 - (uint32_t)P.n_chunk_blocks;
    emit_full_tiles(P, o, (int)f0, (int)(gridDim.x - P.n_seg - P.n_chunk_blocks), L.w);
  }
}

// ----------------------------------------------------------------- one workgroup per segment
// A plan whose segments are all modest (single_segment_ok) is selected after the streaming
// pass by this kernel alone, one workgroup per segment, instead of the chain of kernels over
// candidate chunks (whose launches, not bytes, set such a call's time):
//  * a small segment: select_small, from its residual;
//  * candidates complete (k <= count <= capacity): the tiles' runs placed in index order by a
//    scan in LDS; the exact k-th key by near_select over the candidates (held in registers
//    when they fit one chunk, placed there in index order through LDS; else read from the
//    candidate buffer in any order); then emitted in order, more than one chunk gathered a
//    chunk at a time, each place's run found by bisection over the scan;
//  * otherwise (a miss, an overflow, no estimate yet): a radix select streamed over the
//    segment's residual (three passes), then its tiles emitted in order.
// Then the segment's finish.
constexpr int kSingleTiles = (int)((kSingleMaxElems + kTile - 1) / kTile);

struct alignas(16) SingleLds {
  float val[kChunk];                 // at most one chunk of candidates in index order (then
  int32_t idx[kChunk];               // val holds the select's list of keys)
  uint32_t rdst[kSingleTiles + 1];   // per tile: the index-ordered place of its run (then c)
  uint32_t roff[kSingleTiles];       // per tile: the run's offset in the candidate buffer
  uint32_t n_list;
  SmallLds sm;
};
// Keys the single workgroup's select ranks in its list (held in the value slots).
constexpr uint32_t kSingleList = (uint32_t)kChunk < kListCap ? (uint32_t)kChunk : kListCap;

// The k-th largest key of a key source by a radix select, digits of 11, 11 and 9 bits, each
// LDS histogram (zero on entry and on return) cleared by its digit search; *ties: the entries
// to take at exactly the k-th key.  each(f) calls f(key) for the source's keys, each thread a
// share.  False when the source holds fewer than k keys.  Contains barriers.
template <typename Each>
__device__ __forceinline__ bool radix_select(Each each, uint32_t k, SmallLds& L,
                                             uint32_t* kth, uint32_t* ties) {
  uint32_t prefix = 0, kk = k;
  for (int pass = 0; pass < 3; ++pass) {
    const uint32_t pm = prefix_mask(pass), dm = digit_mask(pass);
    const int sh = digit_shift(pass);
    each([&](uint32_t key) {
      if ((key & pm) == prefix) atomicAdd(&L.h[(key >> sh) & dm], 1u);
    });
    __syncthreads();
    uint32_t d, above, bin;
    if (!find_digit<true>(L.h, kk, L.tmp, L.out, &d, &above, &bin)) return false;
    prefix |= d << sh;
    kk -= above;
  }
  *kth = prefix;
  *ties = kk;
  return true;
}

__global__ __launch_bounds__(kThreads) void k_single(DevPlan P, const float* __restrict__ e,
                                                    EmitOut o) {
  __shared__ SingleLds L;
  const int s = blockIdx.x;
  const uint32_t k = call_k(P, s);
  const int64_t s0 = P.seg_off[s];
  const int32_t n_s = (int32_t)(P.seg_off[s + 1] - s0);
  const int64_t t0 = P.tile_base[s];
  const int nt = (int)(P.tile_base[s + 1] - t0);
  const uint32_t thr_used = capture_thr(P, s);
  const uint32_t c = P.cand_cnt[s];
  const int pb = slot_base();
  for (int i = threadIdx.x; i < kHistBins; i += kThreads) L.sm.h[i] = 0;
  __syncthreads();
  if (k == 0) {   // uniform
    if (threadIdx.x == 0) P.mode[s] = kModeSkip;
    finalize_segment(P, o, s, 0u, kModeSkip, false, thr_used, c, 0u, 0u, 0u, 0u);
    return;
  }
  if (P.seg_flags[s] & kSegSmall) {   // uniform
    uint32_t kth, ties, mx;
    select_small(P, e, o, s, k, L.sm, &kth, &ties, &mx);
    if (threadIdx.x == 0) {
      P.mode[s] = kModeSmall;
      if (P.scales) P.scales[s] = __uint_as_float(mx) / 127.0f;
      P.kth[s] = kth;
      P.ties[s] = ties;
    }
    __syncthreads();   // every thread has read k (the threshold call's count) before it is reset
    finalize_segment(P, o, s, k, kModeSmall, false, thr_used, c, 0u, kth, ties, mx);
    if (threadIdx.x == 0) P.tau_cnt[s] = 0;
    return;
  }
  EmitOut os = o;
  if (os.rk_scale) os.vmul = os.rk_scale[s];
  if (os.vsrc_scale) os.gmul = os.vsrc_scale[s];
  const bool want_mx = P.scales || os.codes;
  const bool pend = seg_pending(P, s);
  uint32_t kth = 0, ties = 0, mx = 0, c_sel = 0, mode;
  uint32_t bad = 0;
  if (!pend) {   // uniform
    mode = kModeCand;
    c_sel = c;
    const int64_t cb = P.cand_base[s];
    const bool one = c <= (uint32_t)kChunk;
    // one chunk of candidates: their loads issued before the scan below (they do not wait on
    // it), placed after it
    constexpr int kPer = kChunk / kThreads;
    float cv[kPer];
    int32_t ci[kPer];
    if (one) {   // uniform
#pragma unroll
      for (int q = 0; q < kPer; ++q) {
        const uint32_t j = threadIdx.x + (uint32_t)(q * kThreads);
        cv[q] = j < c ? P.cand_val[cb + j] : 0.0f;
        ci[q] = j < c ? P.cand_idx[cb + j] : -1;
      }
    }
    // the runs' places in index order: an exclusive scan of the run sizes over the tiles
    uint32_t carry = 0;
    for (int tb = 0; tb < nt; tb += kThreads) {
      const int lt = tb + (int)threadIdx.x;
      const uint32_t n = lt < nt ? P.run_cnt[t0 + lt] : 0u;
      uint32_t tot;
      const uint32_t d = carry + block_excl_scan<kThreads>(n, L.sm.tmp, &tot);
      if (lt < nt) {
        L.rdst[lt] = d;
        L.roff[lt] = P.run_off[t0 + lt];
      }
      carry += tot;
    }
    if (threadIdx.x == 0) L.rdst[nt] = carry;
    __syncthreads();
    // the candidates at index-ordered places base + p of a tile-shaped block: each place's
    // run found by bisection over the scan (rdst[t] <= place < rdst[t + 1]); a place outside
    // the buffer's c entries, or an index outside its run's tile, marks the call bad
    f4 x[kSlots];
    i4 ix[kSlots];
    auto gather = [&](uint32_t base, int len) {
      uint32_t b = 0;
#pragma unroll
      for (int v = 0; v < kSlots; ++v)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int p = pb + v * 256 + q;
          float val = 0.0f;
          int32_t id = 0;
          if (p < len) {
            const uint32_t pos = base + (uint32_t)p;
            int lo = 0, hi = nt;
            while (hi - lo > 1) {
              const int mid = (lo + hi) >> 1;
              if (L.rdst[mid] <= pos) lo = mid; else hi = mid;
            }
            const uint32_t off = L.roff[lo] + (pos - L.rdst[lo]);
            if (off < c) {
              val = P.cand_val[cb + off];
              id = P.cand_idx[cb + off];
            }
            if (off >= c || id < lo * kTile || id >= min((lo + 1) * kTile, n_s)) {
              b = 1;
              id = 0;
            }
          }
          x[v][q] = val;
          ix[v][q] = id;
        }
      return block_max<kThreads>(b, L.sm.tmp);
    };
    // the keys: one chunk from registers, more read from the candidate buffer in any order
    auto reg_keys = [&](auto f) {
#pragma unroll
      for (int v = 0; v < kSlots; ++v)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (pb + v * 256 + q < (int)c) f(mag_key(x[v][q]));
    };
    auto buf_keys = [&](auto f) {
      for (uint32_t base = 0; base < c; base += (uint32_t)kChunk) {
        const int len = (int)min((uint32_t)kChunk, c - base);
        f4 y[kSlots];
        load_tile(P.cand_val + cb + base, len, y);
#pragma unroll
        for (int v = 0; v < kSlots; ++v)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (pb + v * 256 + q < len) f(mag_key(y[v][q]));
      }
    };
    bad = carry != c;   // uniform
    if (!bad && one) {   // uniform: placed in LDS, each candidate at its run's place
#pragma unroll
      for (int q = 0; q < kPer; ++q) {
        const uint32_t j = threadIdx.x + (uint32_t)(q * kThreads);
        if (j >= c) break;
        const float v = cv[q];
        const int32_t id = ci[q];
        const int lt = id >= 0 && id < n_s ? id / kTile : -1;
        uint32_t dst = (uint32_t)kChunk;
        if (lt >= 0 && lt < nt && j >= L.roff[lt]) dst = L.rdst[lt] + (j - L.roff[lt]);
        if (dst < c) {
          L.val[dst] = v;
          L.idx[dst] = id;
        } else {
          bad = 1;
        }
      }
      bad = block_max<kThreads>(bad, L.sm.tmp);   // (its barriers order the LDS writes above)
#pragma unroll
      for (int v = 0; v < kSlots; ++v)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int p = pb + v * 256 + q;
          x[v][q] = p < (int)c ? L.val[p] : 0.0f;
        }
    }
    bool ok = false;
    if (!bad) {   // uniform
      // the candidates' windowed histogram from the capture floor, as the chain's scatter
      const bool window = P.keys == kKeysMagnitude && thr_used > 0;
      const NearLds nl{L.sm.h, L.sm.tmp, L.sm.out, &L.n_list,
                       reinterpret_cast<uint32_t*>(L.val), kSingleList};
      ok = one ? near_select(reg_keys, thr_used, 0x7FFFFFFFu, window, k, nl, &kth, &ties, &mx)
               : near_select(buf_keys, thr_used, 0x7FFFFFFFu, window, k, nl, &kth, &ties, &mx);
      if (want_mx) mx = block_max<kThreads>(mx, L.sm.tmp);
    }
    if (ok) {   // uniform
      if (os.codes) os.scale = __uint_as_float(mx) / 127.0f;
      // emitted a chunk at a time in index order, the ties kept counted across chunks
      uint32_t eqb = 0, kept = 0;
      for (uint32_t base = 0; base < c; base += (uint32_t)kChunk) {
        const int len = (int)min((uint32_t)kChunk, c - base);
        if (!one && gather(base, len)) {   // uniform
          bad = 1;
          break;
        }
        auto slot_idx = [&](int v) {
          if (!one) return ix[v];
          i4 r;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int p = pb + v * 256 + q;
            r[q] = p < (int)c ? L.idx[p] : 0;
          }
          return r;
        };
        uint32_t gt, eq;
        count_block(x, len, kth, L.sm.tmp, &gt, &eq);
        emit_block(x, len, slot_idx, kth, ties, eqb, eq, P.out_off[s] + kept, P.out_off[s + 1],
                   s0, n_s, L.sm.w, os);
        kept += gt + (eqb < ties ? min(eq, ties - eqb) : 0u);
        eqb += eq;
      }
      if (threadIdx.x == 0 && !bad && kept != k) atomicOr(P.err, 2u);
    } else {
      bad = 1;
    }
  } else {
    // no complete candidates: a radix select streamed over the segment's residual, then its
    // tiles emitted in order
    mode = kModeFull;
    auto seg_keys = [&](auto f) {   // two tiles' loads in flight at a time
      for (int j = 0; j < nt; j += 2) {
        int64_t st0, st1 = 0;
        int len0, len1 = 0;
        tile_range(P, s, t0 + j, &st0, &len0);
        if (j + 1 < nt) tile_range(P, s, t0 + j + 1, &st1, &len1);
        f4 x0[kSlots], x1[kSlots];
        key_tile(P, e, st0, len0, x0);
        key_tile(P, e, st1, len1, x1);
#pragma unroll
        for (int v = 0; v < kSlots; ++v)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            if (pb + v * 256 + q < len0) f(mag_key(x0[v][q]));
            if (pb + v * 256 + q < len1) f(mag_key(x1[v][q]));
          }
      }
    };
    const bool ok = radix_select(seg_keys, k, L.sm, &kth, &ties);
    if (want_mx) {   // uniform
      seg_keys([&](uint32_t key) { mx = max(mx, key); });
      mx = block_max<kThreads>(mx, L.sm.tmp);
    }
    if (ok) {   // uniform
      if (os.codes) os.scale = __uint_as_float(mx) / 127.0f;
      uint32_t eqb = 0, kept = 0;
      f4 xn[kSlots];   // the next tile's keys, loaded while this one is emitted
      int64_t stn;
      int lenn;
      tile_range(P, s, t0, &stn, &lenn);
      key_tile(P, e, stn, lenn, xn);
      for (int j = 0; j < nt; ++j) {
        f4 x[kSlots];
#pragma unroll
        for (int v = 0; v < kSlots; ++v) x[v] = xn[v];
        const int len = lenn;
        if (j + 1 < nt) {
          tile_range(P, s, t0 + j + 1, &stn, &lenn);
          key_tile(P, e, stn, lenn, xn);
        }
        uint32_t gt, eq;
        count_block(x, len, kth, L.sm.tmp, &gt, &eq);
        emit_seg_tile(P, os, s, t0 + j, kth, ties, eqb, eq, kept, x, L.sm.w);
        kept += gt + (eqb < ties ? min(eq, ties - eqb) : 0u);
        eqb += eq;
      }
      if (threadIdx.x == 0 && kept != k) atomicOr(P.err, 2u);
    } else {
      bad = 1;
    }
  }
  if (threadIdx.x == 0) {
    if (bad) atomicOr(P.err, 16u);
    P.mode[s] = mode;
  }
  finalize_segment(P, o, s, k, mode, pend, thr_used, c, c_sel, kth, ties, mx);
}

// -------------------------------------------------------------------------------- Random-k
// Random-k ("Gradient Compression", memory-compression glossary, Random-k section): exactly k
// positions per segment, those with the k largest random keys (rand_key_tile), a uniformly
// random subset drawn anew each step.  The streaming pass forms acc as the Top-k pass does and
// captures by key instead of magnitude; the select and the ordered emit are shared, the kept
// values then read back from where acc lives.

template <bool kMomentum, bool kEF, bool kScale = false>
__global__ __launch_bounds__(kThreads) void k_randk_capture(DevPlan P, const float* __restrict__ g,
                                                           float* __restrict__ e,
                                                           float* __restrict__ u, float m) {
  __shared__ uint32_t s_w[kWaves];
  __shared__ uint32_t s_base;
  const int64_t t = blockIdx.x;
  const int4 desc = P.tile_desc[t];
  const int64_t start = (int64_t)(((uint64_t)(uint32_t)desc.y << 32) | (uint32_t)desc.x);
  const int len = desc.z, s = desc.w;
  const uint32_t thr = P.thr[s];  // kNoCapture: this segment takes the exact fallback
  const float gf = kScale ? P.gscale[s] : 1.0f;
  reset_call_lists(P);
  f4 key[kSlots];
  if (kEF && len == kTile && (start & 3) == 0) {
    // whole aligned tile: issue the loads, draw the keys while they are in flight
    const int pb = slot_base();
    const f4* g4 = reinterpret_cast<const f4*>(g + start);
    f4* e4 = reinterpret_cast<f4*>(e + start);
    f4* u4 = kMomentum ? reinterpret_cast<f4*>(u + start) : nullptr;
    f4 gv[kSlots], ev[kSlots], uv[kSlots];
#pragma unroll
    for (int v = 0; v < kSlots; ++v) {
      const int q = (pb + v * 256) >> 2;
      gv[v] = GC_NT_LOAD_G ? __builtin_nontemporal_load(g4 + q) : g4[q];
      ev[v] = GC_NT_LOAD_E ? __builtin_nontemporal_load(e4 + q) : e4[q];
      if (kMomentum) uv[v] = GC_NT_LOAD_E ? __builtin_nontemporal_load(u4 + q) : u4[q];
    }
    if (thr != kNoCapture) rand_key_tile(P, start, len, key);
#pragma unroll
    for (int v = 0; v < kSlots; ++v) {
      const int q = (pb + v * 256) >> 2;
      f4 x = gv[v] * gf;
      if (kMomentum) {
        const f4 mu = m * uv[v];
        x = mu + x;
        if (GC_NT_STORE_E) __builtin_nontemporal_store(x, u4 + q); else u4[q] = x;
      }
      const f4 a = ev[v] + x;
      if (GC_NT_STORE_E) __builtin_nontemporal_store(a, e4 + q); else e4[q] = a;
    }
  } else {
    if (kEF) {
      f4 acc[kSlots];
      ef_add_tile<kMomentum>(g, gf, e, u, m, start, len, acc);
    } else if (kMomentum) {
      momentum_tile(g, gf, u, m, start, len);
    }  // neither is served by k_randk_keys (nothing to stream; g is read at the kept positions)
    if (thr != kNoCapture) rand_key_tile(P, start, len, key);
  }
  if (thr == kNoCapture) return;  // uniform
  capture_tile(P, s, t, start, len, key, thr, &P.cand_cnt[s], s_w, &s_base);
}

// Random-k without error feedback or momentum reads nothing in its pass: it only draws keys
// and captures the ones at or above the threshold, as k_randk_capture does, with the same
// runs and order.  With no memory stream to hide behind, the workgroup-wide ranks and barriers
// of the tile layout dominate, so here one wave owns a whole tile: slot v (0 .. kTile/256 - 1)
// of lane l holds the 4 elements from v * 256 + l * 4 (index order is slot, lane, element).
// The wave draws its keys slot by slot, ranks the flagged ones with ballots as it goes and
// stages the first kRkStage of them (key, tile offset) in its own LDS rows.  Then the
// workgroup's kRkWaves tiles reserve their runs together, one atomic per segment they cover
// (consecutive tiles, runs in tile order): with one atomic per tile, thousands of waves that
// finish their tiles of one large segment at once contend on the segment's counter.  Each
// wave then copies its staged entries out; entries past the staging rows (dense segments) are
// drawn again from the per-slot flags.  One barrier pair per workgroup.
// Tiles (waves) per workgroup: one reservation for four tiles took the 7B shape's key pass
// from 5.1 to 2.9 ms; eight measured the same, sixteen slower (one workgroup per CU).
constexpr int kRkWaves = 4;
constexpr int kRkSlots = kTile / 256;
constexpr int kRkStage = 256;
// Slots whose keys a wave draws before it looks at their flags (independent Philox chains).
constexpr int kRkGroup = 4;
static_assert(8 % kRkGroup == 0, "groups of slots divide a word of eight");
static_assert(kRkSlots % 8 == 0, "a tile must hold whole words of eight 256-element slots");

// The keys of one tile: per-slot flags (key >= thr) into pk, one nibble per slot, the first
// kRkStage flagged (key, tile offset) pairs into the wave's LDS rows in index order; returns
// the tile's flagged count (wave-uniform).  kWhole: the tile holds kTile elements.  A slot
// where no lane holds two flagged keys (nearly all of them at the usual densities) is ranked
// by one prefix count over the lanes; otherwise by one per element position.
template <bool kAligned, bool kWhole>
__device__ __forceinline__ uint32_t rk_draw(const DevPlan& P, int64_t start, int len,
                                            uint32_t thr, int lane, uint32_t* sk, int32_t* si,
                                            uint32_t (&pk)[kRkSlots / 8]) {
  uint32_t cnt = 0;   // wave-uniform: flagged entries so far
#pragma unroll
  for (int wi = 0; wi < kRkSlots / 8; ++wi) {
    uint32_t word = 0;
#pragma unroll
    for (int j0 = 0; j0 < 8; j0 += kRkGroup) {
      uint32_t k[kRkGroup][4];
      uint32_t gw = 0;
#pragma unroll
      for (int jj = 0; jj < kRkGroup; ++jj) {
        const int p0 = (wi * 8 + j0 + jj) * 256 + lane * 4;
        rand_key4<kAligned>(P, start + p0, k[jj]);
#pragma unroll
        for (int c = 0; c < 4; ++c)
          gw |= ((kWhole || p0 + c < len) && k[jj][c] >= thr) ? (1u << (4 * jj + c)) : 0u;
      }
      word |= gw << (4 * j0);
      if (!__ballot(gw != 0)) continue;   // uniform
#pragma unroll
      for (int jj = 0; jj < kRkGroup; ++jj) {
        const uint32_t nib = (gw >> (4 * jj)) & 0xFu;
        const uint64_t any = __ballot(nib != 0);
        if (!any) continue;   // uniform
        const int p0 = (wi * 8 + j0 + jj) * 256 + lane * 4;
        if (!__ballot((nib & (nib - 1u)) != 0)) {   // uniform: at most one flagged key a lane
          const uint32_t r = cnt + lanes_below(any);
          cnt += __popcll(any);
          if (nib && r < (uint32_t)kRkStage) {   // the lane's one flagged key, chosen by its bit
            sk[r] = (nib & 1u) ? k[jj][0] : (nib & 2u) ? k[jj][1] : (nib & 4u) ? k[jj][2]
                                                                               : k[jj][3];
            si[r] = p0 + (int)__builtin_ctz(nib);
          }
          continue;
        }
        const uint64_t m0 = __ballot(nib & 1u), m1 = __ballot(nib & 2u);
        const uint64_t m2 = __ballot(nib & 4u), m3 = __ballot(nib & 8u);
        uint32_t r = cnt + lanes_below(m0) + lanes_below(m1) + lanes_below(m2) +
                     lanes_below(m3);
        cnt += __popcll(m0) + __popcll(m1) + __popcll(m2) + __popcll(m3);
#pragma unroll
        for (int c = 0; c < 4; ++c)
          if ((nib >> c) & 1u) {
            if (r < (uint32_t)kRkStage) {
              sk[r] = k[jj][c];
              si[r] = p0 + c;
            }
            ++r;
          }
      }
    }
    pk[wi] = word;
  }
  return cnt;
}

// Tile t's run at base: its run record, the staged entries copied out, and the entries past
// the staging rows drawn again from the flags.
template <bool kAligned>
__device__ __forceinline__ void rk_write(const DevPlan& P, int64_t t, int64_t start, int s,
                                         uint32_t base, uint32_t cnt, int lane,
                                         const uint32_t* sk, const int32_t* si,
                                         const uint32_t (&pk)[kRkSlots / 8]) {
  if (lane == 0) {
    P.run_off[t] = base;
    P.run_cnt[t] = cnt;
  }
  if (cnt == 0) return;   // uniform
  const uint32_t cap = P.cand_cap[s];
  float* cv = P.cand_val + P.cand_base[s];
  int32_t* ci = P.cand_idx + P.cand_base[s];
  const int32_t lstart = (int32_t)(start - P.seg_off[s]);
  const uint32_t staged = min(cnt, (uint32_t)kRkStage);
  for (uint32_t i = lane; i < staged; i += 64) {   // the wave's own LDS rows, written above
    const uint32_t q = base + i;
    if (q < cap) {
      cv[q] = __uint_as_float(sk[i]);
      ci[q] = lstart + si[i];
    }
  }
  if (cnt <= (uint32_t)kRkStage) return;   // uniform
  uint32_t run = 0;   // ranks past the staging rows: draw those keys again
#pragma unroll
  for (int wi = 0; wi < kRkSlots / 8; ++wi) {
    const uint32_t word = pk[wi];
    if (!__ballot(word != 0)) continue;   // uniform
    for (int j = 0; j < 8; ++j) {
      const uint32_t nib = (word >> (4 * j)) & 0xFu;
      if (!__ballot(nib != 0)) continue;   // uniform
      const uint64_t m0 = __ballot(nib & 1u), m1 = __ballot(nib & 2u);
      const uint64_t m2 = __ballot(nib & 4u), m3 = __ballot(nib & 8u);
      uint32_t r = run + lanes_below(m0) + lanes_below(m1) + lanes_below(m2) + lanes_below(m3);
      run += __popcll(m0) + __popcll(m1) + __popcll(m2) + __popcll(m3);
      if (!nib || r + (uint32_t)__popc(nib) <= (uint32_t)kRkStage) continue;
      const int p0 = (wi * 8 + j) * 256 + lane * 4;
      uint32_t k[4];
      rand_key4<kAligned>(P, start + p0, k);
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if ((nib >> c) & 1u) {
          const uint32_t q = base + r;
          if (r >= (uint32_t)kRkStage && q < cap) {
            cv[q] = __uint_as_float(k[c]);
            ci[q] = lstart + p0 + c;
          }
          ++r;
        }
    }
  }
}

__global__ __launch_bounds__(kRkWaves * 64) void k_randk_keys(DevPlan P) {
  __shared__ uint32_t s_key[kRkWaves][kRkStage];
  __shared__ int32_t s_idx[kRkWaves][kRkStage];
  __shared__ uint32_t s_cnt[kRkWaves], s_base[kRkWaves];
  __shared__ int32_t s_seg[kRkWaves];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t t = (int64_t)blockIdx.x * kRkWaves + w;
  reset_call_lists(P);
  int s = -1;   // -1: nothing to capture (past the last tile, or a segment without threshold)
  int64_t start = 0;
  uint32_t cnt = 0;
  uint32_t pk[kRkSlots / 8];
  if (t < P.n_tiles) {   // wave-uniform
    const int4 desc = P.tile_desc[t];
    start = (int64_t)(((uint64_t)(uint32_t)desc.y << 32) | (uint32_t)desc.x);
    const int len = desc.z, sd = desc.w;
    const uint32_t thr = P.thr[sd];
    if (thr != kNoCapture) {   // else the segment takes the exact fallback
      s = sd;
      if ((start & 3) == 0 && len == kTile)   // a whole tile, one Philox block per lane
        cnt = rk_draw<true, true>(P, start, len, thr, lane, s_key[w], s_idx[w], pk);
      else if ((start & 3) == 0)
        cnt = rk_draw<true, false>(P, start, len, thr, lane, s_key[w], s_idx[w], pk);
      else
        cnt = rk_draw<false, false>(P, start, len, thr, lane, s_key[w], s_idx[w], pk);
    }
  }
  if (lane == 0) {
    s_cnt[w] = cnt;
    s_seg[w] = s;
  }
  __syncthreads();
  if (threadIdx.x == 0) {   // one reservation per segment covered (its tiles are consecutive)
    for (int i = 0; i < kRkWaves;) {
      const int si = s_seg[i];
      int j = i + 1;
      while (j < kRkWaves && s_seg[j] == si) ++j;
      if (si >= 0) {
        uint32_t tot = 0;
        for (int q = i; q < j; ++q) tot += s_cnt[q];
        uint32_t b = tot ? atomicAdd(&P.cand_cnt[si], tot) : 0u;
        for (int q = i; q < j; ++q) {
          s_base[q] = b;
          b += s_cnt[q];
        }
      }
      i = j;
    }
  }
  __syncthreads();
  if (s < 0) return;   // wave-uniform
  if ((start & 3) == 0)
    rk_write<true>(P, t, start, s, s_base[w], cnt, lane, s_key[w], s_idx[w], pk);
  else
    rk_write<false>(P, t, start, s, s_base[w], cnt, lane, s_key[w], s_idx[w], pk);
}

// Everything after the streaming pass: the per-segment list, the fallback kernels (they end
// at once unless a segment's capture was incomplete), the candidates ordered and ranked, the
// per-segment finish, and the ordered emission with the small segments' selects beside it.
// e holds acc (magnitude keys); Random-k keys are drawn again where needed.
void select_emit(const DevPlan& P, const float* e, const EmitOut& o, hipStream_t st) {
  if (P.single) {
    k_single<<<(unsigned)P.n_seg, kThreads, 0, st>>>(P, e, o);
    return;
  }
  const int64_t nt = P.n_tiles > 0 ? P.n_tiles : 1;
  const unsigned fb = (unsigned)(nt < kFallbackBlocks ? nt : kFallbackBlocks);
  k_list<<<(unsigned)P.n_seg + fb, kThreads, 0, st>>>(P, e);
  k_fb_capture<<<fb, kThreads, 0, st>>>(P, e);
  k_fb_hist2<<<fb, kThreads, 0, st>>>(P, e);
  k_fb_count<<<fb, kThreads, 0, st>>>(P, e);
  if (P.n_chunk_blocks > 0) {
    k_scatter<<<(unsigned)P.n_chunk_blocks, kThreads, 0, st>>>(P);
    k_collect<<<(unsigned)P.n_chunk_blocks, kThreads, 0, st>>>(P);
  }
  k_finish<<<(unsigned)P.n_seg, kThreads, 0, st>>>(P, e, o);
  const unsigned nfull = (unsigned)(nt < kFullBlocks ? nt : kFullBlocks);
  k_emit<<<(unsigned)(P.n_seg + P.n_chunk_blocks) + nfull, kThreads, 0, st>>>(P, e, o);
}

}  // namespace

hipError_t launch_compress(const DevPlan& P0, const float* g, float* e, float* u, float m,
                           float* out_vals, int32_t* out_idx, const Int8Args& q8, bool cold,
                           hipStream_t st, hipEvent_t ev_begin, hipEvent_t ev_end) {
  if (P0.n_seg == 0) return hipSuccess;
  DevPlan P = P0;
  P.codec = kCodecTopk;
  P.keys = kKeysMagnitude;
  P.tau = nullptr;
  P.out_count = nullptr;
  P.scales = q8.enabled ? q8.scales : nullptr;
  if (cold && P.n_sample > 0) {
    if (u)
      k_sample_hist<true><<<(unsigned)P.n_sample, kThreads, 0, st>>>(P, g, e, u, m);
    else
      k_sample_hist<false><<<(unsigned)P.n_sample, kThreads, 0, st>>>(P, g, e, nullptr, m);
    k_sample_decide<<<(unsigned)P.n_seg, kThreads, 0, st>>>(P);
  }
  if (ev_begin) (void)hipEventRecord(ev_begin, st);
  launch_ef_capture(P, g, e, u, m, false, st);
  if (ev_end) (void)hipEventRecord(ev_end, st);
  EmitOut o{};
  o.e = e;
  o.u = (u && (P.flags & kFlagMomentumMask)) ? u : nullptr;
  o.vals = out_vals;
  o.idx = out_idx;
  o.codes = q8.enabled ? q8.codes : nullptr;
  o.scales = q8.scales;
  o.seed_lo = q8.seed_lo;
  o.seed_hi = q8.seed_hi;
  o.step_lo = q8.step_lo;
  o.err = P.err;
  select_emit(P, e, o, st);
  return hipGetLastError();
}

hipError_t launch_threshold(const DevPlan& P0, const float* g, float* e, float* u, float m,
                            const float* tau, float* out_vals, int32_t* out_idx,
                            int32_t* out_count, hipStream_t st, hipEvent_t ev_begin,
                            hipEvent_t ev_end) {
  if (P0.n_seg == 0) return hipSuccess;
  DevPlan P = P0;
  P.codec = kCodecThreshold;
  P.keys = kKeysMagnitude;
  P.tau = tau;
  P.out_count = out_count;
  P.scales = nullptr;
  if (ev_begin) (void)hipEventRecord(ev_begin, st);
  launch_ef_capture(P, g, e, u, m, true, st);

  if (ev_end) (void)hipEventRecord(ev_end, st);
  EmitOut o{};
  o.e = e;
  o.u = (u && (P.flags & kFlagMomentumMask)) ? u : nullptr;
  o.vals = out_vals;
  o.idx = out_idx;
  o.err = P.err;
  select_emit(P, e, o, st);
  return hipGetLastError();
}

hipError_t launch_randk(const DevPlan& P0, const float* g, float* e, float* u, float m,
                        uint64_t seed, uint64_t step, float* out_vals, int32_t* out_idx,
                        hipStream_t st, hipEvent_t ev_begin, hipEvent_t ev_end) {
  if (P0.n_seg == 0) return hipSuccess;
  DevPlan P = P0;
  P.codec = kCodecRandk;
  P.thr = const_cast<uint32_t*>(P0.thr_rand);   // read only in a Random-k call
  P.keys = kKeysRandom;
  P.tau = nullptr;
  P.out_count = nullptr;
  P.scales = nullptr;
  P.seed_lo = (uint32_t)seed;
  P.seed_hi = (uint32_t)(seed >> 32);
  P.step_lo = (uint32_t)step;
  if (ev_begin) (void)hipEventRecord(ev_begin, st);
  if (P.n_tiles > 0) {
    const unsigned nt = (unsigned)P.n_tiles;
    if (P.gscale) {
      if (e && u) k_randk_capture<true, true, true><<<nt, kThreads, 0, st>>>(P, g, e, u, m);
      else if (e) k_randk_capture<false, true, true><<<nt, kThreads, 0, st>>>(P, g, e, nullptr, m);
      else if (u) k_randk_capture<true, false, true><<<nt, kThreads, 0, st>>>(P, g, nullptr, u, m);
      // neither: the capture reads no g (the emit applies the scale to the gathered values)
      else k_randk_keys<<<blocks_for(P.n_tiles, kRkWaves), kRkWaves * 64, 0, st>>>(P);
    } else {
      if (e && u) k_randk_capture<true, true><<<nt, kThreads, 0, st>>>(P, g, e, u, m);
      else if (e) k_randk_capture<false, true><<<nt, kThreads, 0, st>>>(P, g, e, nullptr, m);
      else if (u) k_randk_capture<true, false><<<nt, kThreads, 0, st>>>(P, g, nullptr, u, m);
      else k_randk_keys<<<blocks_for(P.n_tiles, kRkWaves), kRkWaves * 64, 0, st>>>(P);
    }
  }
  if (ev_end) (void)hipEventRecord(ev_end, st);
  EmitOut o{};
  o.e = e;
  o.u = (u && (P.flags & kFlagMomentumMask)) ? u : nullptr;
  o.vals = out_vals;
  o.idx = out_idx;
  o.err = P.err;
  o.vsrc = e ? e : (u ? u : g);
  o.vsrc_scale = (!e && !u) ? P.gscale : nullptr;
  o.rk_scale = e ? nullptr : P.rk_scale;
  select_emit(P, e, o, st);
  return hipGetLastError();
}

hipError_t launch_reset(const DevPlan& P, hipStream_t st) {
  if (P.n_seg == 0) return hipSuccess;
  k_reset<<<blocks_for(P.n_seg, kThreads), kThreads, 0, st>>>(P);
  return hipGetLastError();
}

}  // namespace gc
