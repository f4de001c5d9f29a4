// gc_topk.hip -- gfx950 kernels of the error-feedback Top-k path, and the threshold and
// Random-k sparsifiers that share its select and ordered emission.
//
// Top-k call (one stream, no host round trip):
//   prep        zero the per-call counters
//   ef_capture  the streaming pass over g, e (and u): momentum, EF add, write acc into e,
//               and capture every (acc, index) whose magnitude key reaches the segment's
//               threshold, as one index-ordered run per tile            [HBM-bound]
//   select_init per segment: keep the candidates if they are complete (count in [k, cap]),
//               else list the segment for re-capture or the exact full-segment path
//   recap_*     first-digit histogram of e and capture at the exact bucket floor (only for
//               segments whose candidates were incomplete)
//   hist/find   x3  radix select of the k-th largest key, digits of 11, 11 and 9 bits,
//               LDS histograms; candidates or, on the full path, the whole segment
//   scatter     candidates into ascending index order (runs placed by tile)
//   count/scan/emit  order-preserving compaction: keys above the k-th, then the ties in
//               index order; writes (value, index) and zeroes e (and u) where kept
//   finalize    next threshold estimate = key(beta * kth), beta steered by the last calls
//
// Threshold and Random-k calls run the same select and emit on a per-call copy of the plan
// (their own k and capture threshold); Random-k ranks per-element Philox keys instead of
// magnitudes.  The two-pass codecs are in gc_codecs.hip, the payload scatters (int8 stage,
// decompression) in gc_scatter.hip, the shared device helpers in gc_device.h.
//
// The method is the Top-K with error feedback of "Communication Optimization > Gradient
// Compression" (Top-K section equations); momentum correction per the "Gradient
// Sparsification" glossary; the int8 stage per the "Gradient Compression" glossary
// (Top-k then 8-bit) with stochastic rounding (QSGD paragraph) and one scale per layer.
#include "gc_device.h"

#pragma clang fp contract(off)

namespace gc {
namespace {

// ------------------------------------------------------------------------------ prep
__global__ __launch_bounds__(kThreads) void k_prep(DevPlan P) {
  const int s = blockIdx.x * kThreads + threadIdx.x;
  if (s < P.n_seg) P.cand_cnt[s] = 0;
  if (s == 0) {
    *P.full_count = 0;
    *P.recap_count = 0;
    *P.act_count = 0;
    *P.err = 0;
  }
}

__global__ __launch_bounds__(kThreads) void k_reset(DevPlan P) {
  const int s = blockIdx.x * kThreads + threadIdx.x;
  if (s < P.n_seg) {   // as on a fresh plan: no estimate, first margins
    P.thr[s] = P.thr_init[s];
    P.thr_est[s] = kNoCapture;
    P.beta[s] = kInitialBeta;
    P.beta_est[s] = kInitialBeta;
  }
}

// Threshold and Random-k calls: this call's k (the plan's, reduced after the capture for a
// threshold call) and capture threshold: for a threshold call max(key(|tau|), floor), the floor
// being the estimate of the k-th largest key kept from the last threshold calls (the capture
// then stays within capacity when more than k entries reach tau); for Random-k the plan's.
__global__ __launch_bounds__(kThreads) void k_prep_call(DevPlan P, const float* __restrict__ tau) {
  const int s = blockIdx.x * kThreads + threadIdx.x;
  if (s < P.n_seg) {
    P.cand_cnt[s] = 0;
    P.k_call[s] = P.k[s];
    if (tau) {
      const uint32_t tk = mag_key(tau[s]), fl = P.thr_est[s];
      P.tau_key[s] = tk;
      P.tau_cnt[s] = 0;
      P.thr_call[s] = fl == kNoCapture ? tk : max(tk, fl);
    } else {
      P.thr_call[s] = P.thr_rand[s];
    }
  }
  if (s == 0) {
    *P.full_count = 0;
    *P.recap_count = 0;
    *P.act_count = 0;
    *P.err = 0;
  }
}

// Threshold call: keep min(number of keys at or above key(|tau|), k) entries per segment (the
// capture counted them all, also above a floor and past the candidate capacity).  The
// candidates, captured at max(key(|tau|), floor), then hold them iff at least that many were
// captured; otherwise the segment takes the exact fallback.
__global__ __launch_bounds__(kThreads) void k_thresh_k(DevPlan P, int32_t* __restrict__ count) {
  const int s = blockIdx.x * kThreads + threadIdx.x;
  if (s >= P.n_seg) return;
  const uint32_t kk = min(P.tau_cnt[s], P.k[s]);
  P.k_call[s] = kk;
  if (count) count[s] = (int32_t)kk;
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
// reaches thr: one atomic on the segment's counter reserves the tile's run; entries past the
// capacity are counted but not stored (the segment then leaves the candidate path).
__device__ __forceinline__ void capture_tile(const DevPlan& P, int s, int64_t t, int64_t start,
                                             int len, const f4 (&acc)[kSlots], uint32_t thr,
                                             uint32_t* s_w, uint32_t* s_base) {
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
    const uint32_t base = total ? atomicAdd(&P.cand_cnt[s], total) : 0u;
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

// -------------------------------------------------------------------------- ef_capture
// One tile per workgroup.  acc = e + (u = m*u + g | g) is written back into e; elements
// whose key reaches the segment's threshold are captured (capture_tile).
// kCountTau (threshold calls): also count the tile's keys >= key(|tau|) into tau_cnt.
// kScale: the plan carries a gradient scale (a separate instantiation, so that the unscaled
// pass has no dependent load of the factor in front of its stream).
template <bool kMomentum, bool kCountTau = false, bool kScale = false>
__global__ __launch_bounds__(kThreads) void k_ef_capture(DevPlan P, const float* __restrict__ g,
                                                        float* __restrict__ e,
                                                        float* __restrict__ u, float m) {
  __shared__ uint32_t s_w[kWaves];
  __shared__ uint32_t s_base;
  __shared__ uint32_t s_tau[kWaves];
#if GC_XCD_REMAP
  // workgroups go round-robin to the 8 XCDs: give XCD x a contiguous range of tiles
  const int64_t G = gridDim.x, per = G / 8, rem = G % 8, xcd = blockIdx.x % 8;
  const int64_t t = xcd * per + (xcd < rem ? xcd : rem) + blockIdx.x / 8;
#else
  const int64_t t = blockIdx.x;
#endif
  const int4 desc = P.tile_desc[t];  // one load: no dependent lookups before the stream
  const int64_t start = (int64_t)(((uint64_t)(uint32_t)desc.y << 32) | (uint32_t)desc.x);
  const int len = desc.z, s = desc.w;
  const int pb = slot_base();
  const float gf = kScale ? P.gscale[s] : 1.0f;

  f4 acc[kSlots];
  if (len == kTile && (start & 3) == 0) {
    const f4* g4 = reinterpret_cast<const f4*>(g + start);
    f4* e4 = reinterpret_cast<f4*>(e + start);
    f4* u4 = kMomentum ? reinterpret_cast<f4*>(u + start) : nullptr;
    f4 gv[kSlots], uv[kSlots];
#pragma unroll
    for (int v = 0; v < kSlots; ++v) {
      const int q = (pb + v * 256) >> 2;
      gv[v] = GC_NT_LOAD_G ? __builtin_nontemporal_load(g4 + q) : g4[q];
      acc[v] = GC_NT_LOAD_E ? __builtin_nontemporal_load(e4 + q) : e4[q];
      if (kMomentum) uv[v] = GC_NT_LOAD_E ? __builtin_nontemporal_load(u4 + q) : u4[q];
    }
#pragma unroll
    for (int v = 0; v < kSlots; ++v) {
      const int q = (pb + v * 256) >> 2;
      f4 x = gv[v] * gf;
      if (kMomentum) {
        const f4 mu = m * uv[v];
        x = mu + x;
        if (GC_NT_STORE_E) __builtin_nontemporal_store(x, u4 + q); else u4[q] = x;
      }
      acc[v] = acc[v] + x;
      if (GC_NT_STORE_E) __builtin_nontemporal_store(acc[v], e4 + q); else e4[q] = acc[v];
    }
  } else {
#pragma unroll
    for (int v = 0; v < kSlots; ++v)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int p = pb + v * 256 + c;
        float a = 0.0f;
        if (p < len) {
          const int64_t i = start + p;
          float x = g[i] * gf;
          if (kMomentum) {
            const float mu = m * u[i];
            x = mu + x;
            u[i] = x;
          }
          a = e[i] + x;
          e[i] = a;
        }
        acc[v][c] = a;
      }
  }
  if (kCountTau) {
    const uint32_t tk = P.tau_key[s];
    uint32_t c = 0;
#pragma unroll
    for (int v = 0; v < kSlots; ++v)
#pragma unroll
      for (int cc = 0; cc < 4; ++cc)
        c += (pb + v * 256 + cc < len && mag_key(acc[v][cc]) >= tk) ? 1u : 0u;
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) c += __shfl_xor(c, d, 64);
    if (lane_id() == 0) s_tau[wave_id()] = c;
    __syncthreads();
    if (threadIdx.x == 0) {
      uint32_t tot = 0;
#pragma unroll
      for (int i = 0; i < kWaves; ++i) tot += s_tau[i];
      if (tot) atomicAdd(&P.tau_cnt[s], tot);
    }
  }
  const uint32_t thr = P.thr[s];
  if (thr == kNoCapture) return;  // uniform: this segment re-captures later
  capture_tile(P, s, t, start, len, acc, thr, s_w, &s_base);
}

// ------------------------------------------------------------------------- select_init
// Per segment: are the captured candidates complete?  Complete means at least k of them
// and none lost to the capacity; then every key >= the k-th largest was captured.
__global__ __launch_bounds__(kThreads) void k_select_init(DevPlan P) {
  const int s = blockIdx.x;
  const uint32_t k = P.k[s], thr = P.thr[s], c = P.cand_cnt[s], cap = P.cand_cap[s];
  uint32_t mode, why = kWhyNone;
  if (k == 0) {
    mode = kModeSkip;
  } else if (thr != kNoCapture && c >= k && c <= cap && !(P.flags & kFlagForceFull)) {
    mode = kModeCand;
  } else {
    mode = kModePending;
    why = thr == kNoCapture ? kWhyCold : (c < k ? kWhyMiss : kWhyOverflow);
  }
  if (threadIdx.x == 0) {
    P.mode[s] = mode;
    P.why[s] = why;
    P.prefix[s] = 0;
    P.kk[s] = k;
    P.kth[s] = 0;
    P.ties[s] = 0;
    if (mode == kModePending) P.recap_list[atomicAdd(P.recap_count, 1u)] = (uint32_t)s;
  }
  if (mode == kModeSkip) return;
  uint32_t* h = P.hist + (size_t)s * 3 * kHistBins;
  for (int i = threadIdx.x; i < 3 * kHistBins; i += kThreads) h[i] = 0;
}

__device__ __forceinline__ int digit_shift(int pass) { return pass == 0 ? 20 : (pass == 1 ? 9 : 0); }
__device__ __forceinline__ uint32_t digit_mask(int pass) { return pass == 2 ? 0x1FFu : 0x7FFu; }
__device__ __forceinline__ uint32_t prefix_mask(int pass) {
  return pass == 0 ? 0u : (pass == 1 ? 0x7FF00000u : 0x7FFFFE00u);
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

// Histogram of one digit over every tile of the listed segments (values read from e).
__device__ void hist_listed_tiles(const DevPlan& P, const float* __restrict__ e,
                                  const uint32_t* list, uint32_t count, uint32_t want_mode,
                                  int pass, int fb, uint32_t* h) {
  for (uint32_t li = 0; li < count; ++li) {
    const int s = (int)list[li];
    if (P.mode[s] != want_mode) continue;
    const uint32_t prefix = P.prefix[s];
    uint32_t* gh = P.hist + ((size_t)s * 3 + pass) * kHistBins;
    for (int64_t t = P.tile_base[s] + fb; t < P.tile_base[s + 1]; t += kFullBlocks) {
      int64_t start;
      int len;
      tile_range(P, s, t, &start, &len);
      for (int i = threadIdx.x; i < kHistBins; i += kThreads) h[i] = 0;
      f4 x[kSlots];
      key_tile(P, e, start, len, x);
      __syncthreads();
      hist_add(h, x, len, prefix, pass);
      __syncthreads();
      hist_flush(h, gh);
      __syncthreads();
    }
  }
}

// ----------------------------------------------------------------------------- recapture
// First-digit histogram of the segments whose candidates were not complete.
__global__ __launch_bounds__(kThreads) void k_recap_hist(DevPlan P, const float* __restrict__ e) {
  __shared__ uint32_t h[kHistBins];
  hist_listed_tiles(P, e, P.recap_list, *P.recap_count, kModePending, 0, blockIdx.x, h);
}

// Digit of the k-th largest key in a histogram (descending scan): d and the count above it.
// s_tmp: __shared__ uint32_t[kWaves]; s_out: __shared__ uint32_t[2].  Contains barriers.
__device__ bool find_digit(const uint32_t* gh, uint32_t kk, uint32_t* s_tmp, uint32_t* s_out,
                           uint32_t* d_out, uint32_t* above_out, uint32_t* bin_out) {
  constexpr int kPer = kHistBins / kThreads;
  uint32_t loc[kPer];
  uint32_t sum = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    loc[j] = gh[kHistBins - 1 - (threadIdx.x * kPer + j)];
    sum += loc[j];
  }
  if (threadIdx.x == 0) {
    s_out[0] = 0xFFFFFFFFu;
    s_out[1] = 0;
    s_out[2] = 0;
  }
  uint32_t tot;
  uint32_t acc = block_excl_scan<kThreads>(sum, s_tmp, &tot);
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    if (acc < kk && acc + loc[j] >= kk) {
      s_out[0] = kHistBins - 1 - (threadIdx.x * kPer + j);
      s_out[1] = acc;
      s_out[2] = loc[j];
    }
    acc += loc[j];
  }
  __syncthreads();
  *d_out = s_out[0];
  *above_out = s_out[1];
  *bin_out = s_out[2];
  return s_out[0] != 0xFFFFFFFFu;
}

// Per pending segment: the first digit of the k-th largest key.  If the keys at or above
// that bucket's floor fit the capacity, they are re-captured (kModeRecap); otherwise the
// segment runs the radix select over all its elements (kModeFull).  Pass 0 is done here.
__global__ __launch_bounds__(kThreads) void k_recap_decide(DevPlan P) {
  __shared__ uint32_t s_tmp[kWaves];
  __shared__ uint32_t s_out[3];
  const int s = blockIdx.x;
  if (P.mode[s] != kModePending) return;
  const uint32_t k = P.k[s];
  uint32_t d, above, bin;
  const bool ok = find_digit(P.hist + (size_t)s * 3 * kHistBins, k, s_tmp, s_out, &d, &above,
                             &bin);
  if (threadIdx.x != 0) return;
  if (!ok) {
    atomicOr(P.err, 1u);
    P.mode[s] = kModeSkip;
    return;
  }
  P.prefix[s] = d << 20;
  P.kk[s] = k - above;
  if (!(P.flags & kFlagForceFull) && above + bin <= P.cand_cap[s]) {
    P.mode[s] = kModeRecap;
    P.thr[s] = d << 20;
    P.cand_cnt[s] = 0;
  } else {
    P.mode[s] = kModeFull;
    P.full_list[atomicAdd(P.full_count, 1u)] = (uint32_t)s;
  }
}

// Re-capture from e (which holds acc) at the exact bucket floor.
__global__ __launch_bounds__(kThreads) void k_recapture(DevPlan P, const float* __restrict__ e) {
  __shared__ uint32_t s_w[kWaves];
  __shared__ uint32_t s_base;
  const uint32_t count = *P.recap_count;
  for (uint32_t li = 0; li < count; ++li) {
    const int s = (int)P.recap_list[li];
    if (P.mode[s] != kModeRecap) continue;
    const uint32_t thr = P.thr[s];
    for (int64_t t = P.tile_base[s] + blockIdx.x; t < P.tile_base[s + 1]; t += kFullBlocks) {
      int64_t start;
      int len;
      tile_range(P, s, t, &start, &len);
      f4 x[kSlots];
      key_tile(P, e, start, len, x);
      capture_tile(P, s, t, start, len, x, thr, s_w, &s_base);
      __syncthreads();
    }
  }
}

__device__ __forceinline__ bool has_candidates(uint32_t mode) {
  return mode == kModeCand || mode == kModeRecap;
}

// Per segment with candidates: index-ordered destination of every tile's run (exclusive
// scan of the run sizes over the segment's tiles).
// Also appends the segment's chunks that hold candidates to the call's list of active chunks
// (the later chunk kernels walk that list instead of every chunk of the capacity).
__global__ __launch_bounds__(1024) void k_runs(DevPlan P) {
  __shared__ uint32_t s_tmp[16];
  __shared__ uint32_t s_act;
  const int s = blockIdx.x;
  if (!has_candidates(P.mode[s])) return;
  const int64_t t0 = P.tile_base[s], t1 = P.tile_base[s + 1];
  uint32_t carry = 0;
  for (int64_t tb = t0; tb < t1; tb += 1024) {
    const int64_t t = tb + threadIdx.x;
    const uint32_t n = t < t1 ? P.run_cnt[t] : 0u;
    uint32_t tot;
    const uint32_t ex = block_excl_scan<1024>(n, s_tmp, &tot);
    if (t < t1) P.run_dst[t] = carry + ex;
    carry += tot;
  }
  const int64_t c0 = P.chunk_base[s];
  const uint32_t na = (uint32_t)min(((int64_t)P.cand_cnt[s] + kChunk - 1) / kChunk,
                                    P.chunk_base[s + 1] - c0);
  if (threadIdx.x == 0) s_act = na ? atomicAdd(P.act_count, na) : 0u;
  __syncthreads();
  for (uint32_t j = threadIdx.x; j < na; j += 1024) P.act_chunk[s_act + j] = (uint32_t)(c0 + j);
}

// ------------------------------------------------------------------------------ scatter
// Candidates into ascending index order (tile t's run goes to run_dst[t]); on the estimate
// path, also the first-digit histogram of the candidates.  One chunk; contains barriers.
__device__ void scatter_chunk(const DevPlan& P, int64_t ch, uint32_t* h, uint32_t* s_m) {
  const int s = P.chunk_seg[ch];
  const uint32_t mode = P.mode[s];
  if (!has_candidates(mode)) return;
  const int64_t c = P.cand_cnt[s];
  const int64_t j0 = (ch - P.chunk_base[s]) * (int64_t)kChunk;
  if (j0 >= c) return;
  const bool do_hist = mode == kModeCand;
  if (do_hist)
    for (int i = threadIdx.x; i < kHistBins; i += kThreads) h[i] = 0;
  const int len = (int)min((int64_t)kChunk, c - j0);
  const int64_t cb = P.cand_base[s], tb = P.tile_base[s];
  constexpr int kPer = kChunk / kThreads;
  int32_t ix[kPer];
  float vx[kPer];
#pragma unroll
  for (int r = 0; r < kPer; ++r) {
    const int p = r * kThreads + threadIdx.x;
    ix[r] = p < len ? P.cand_idx[cb + j0 + p] : 0;
    vx[r] = p < len ? P.cand_val[cb + j0 + p] : 0.0f;
  }
  if (do_hist) __syncthreads();
#pragma unroll
  for (int r = 0; r < kPer; ++r) {
    const int p = r * kThreads + threadIdx.x;
    if (p < len) {
      const int64_t t = tb + ix[r] / kTile;
      const uint32_t dst = P.run_dst[t] + ((uint32_t)(j0 + p) - P.run_off[t]);
      if (ix[r] >= 0 && t < P.tile_base[s + 1] && dst < (uint32_t)c) {
        P.sort_val[cb + dst] = vx[r];
        P.sort_idx[cb + dst] = ix[r];
      } else {
        atomicOr(P.err, 8u);
      }
      if (do_hist) atomicAdd(&h[mag_key(vx[r]) >> 20], 1u);
    }
  }
  uint32_t mx = 0;
#pragma unroll
  for (int r = 0; r < kPer; ++r)
    if (r * kThreads + (int)threadIdx.x < len) mx = max(mx, mag_key(vx[r]));
  mx = block_max<kThreads>(mx, s_m);
  if (threadIdx.x == 0) P.chunk_max[ch] = mx;
  if (do_hist) {
    __syncthreads();
    hist_flush(h, P.hist + (size_t)s * 3 * kHistBins);
  }
}

// The workgroups walk the call's list of chunks that hold candidates.
__global__ __launch_bounds__(kThreads) void k_scatter(DevPlan P) {
  __shared__ uint32_t h[kHistBins];
  __shared__ uint32_t s_m[kWaves];
  const uint32_t na = *P.act_count;
  for (uint32_t i = blockIdx.x; i < na; i += (uint32_t)P.n_chunk_blocks) {
    scatter_chunk(P, P.act_chunk[i], h, s_m);
    __syncthreads();   // the next chunk reuses h
  }
}

// --------------------------------------------------------------------------------- hist
// Passes 1 and 2.  Workgroups [0, n_chunk_blocks) histogram the sorted candidate chunks of the
// call's active list; the last kFullBlocks the tiles of the segments on the full path.
__device__ void hist_chunk(const DevPlan& P, int64_t ch, int pass, uint32_t* h) {
  const int s = P.chunk_seg[ch];
  if (!has_candidates(P.mode[s])) return;
  const int64_t c = P.cand_cnt[s];
  const int64_t j0 = (ch - P.chunk_base[s]) * (int64_t)kChunk;
  if (j0 >= c) return;
  const int len = (int)min((int64_t)kChunk, c - j0);
  const uint32_t prefix = P.prefix[s];
  for (int i = threadIdx.x; i < kHistBins; i += kThreads) h[i] = 0;
  f4 x[kSlots];
  load_tile(P.sort_val + P.cand_base[s] + j0, len, x);
  __syncthreads();
  hist_add(h, x, len, prefix, pass);
  __syncthreads();
  hist_flush(h, P.hist + ((size_t)s * 3 + pass) * kHistBins);
}

__global__ __launch_bounds__(kThreads) void k_hist(DevPlan P, const float* __restrict__ e,
                                                   int pass) {
  __shared__ uint32_t h[kHistBins];
  if (blockIdx.x < (uint32_t)P.n_chunk_blocks) {
    const uint32_t na = *P.act_count;
    for (uint32_t i = blockIdx.x; i < na; i += (uint32_t)P.n_chunk_blocks) {
      hist_chunk(P, P.act_chunk[i], pass, h);
      __syncthreads();   // the next chunk reuses h
    }
    return;
  }
  hist_listed_tiles(P, e, P.full_list, *P.full_count, kModeFull, pass,
                    blockIdx.x - P.n_chunk_blocks, h);
}

// --------------------------------------------------------------------------------- find
// Per segment: the digit of this pass that holds the kk-th largest key of the prefix.
// Pass 0 only for the estimate path (the others took it in k_recap_decide).
__global__ __launch_bounds__(kThreads) void k_find(DevPlan P, int pass) {
  __shared__ uint32_t s_tmp[kWaves];
  __shared__ uint32_t s_out[3];
  const int s = blockIdx.x;
  const uint32_t mode = P.mode[s];
  if (mode == kModeSkip || (pass == 0 && mode != kModeCand)) return;
  const uint32_t kk = P.kk[s];
  uint32_t d, above, bin;
  const bool ok = find_digit(P.hist + ((size_t)s * 3 + pass) * kHistBins, kk, s_tmp, s_out, &d,
                             &above, &bin);
  if (threadIdx.x != 0) return;
  if (!ok) {  // cannot happen when the histogram holds >= kk keys
    atomicOr(P.err, 1u);
    return;
  }
  const uint32_t prefix = P.prefix[s] | (d << digit_shift(pass));
  const uint32_t nk = kk - above;
  P.prefix[s] = prefix;
  P.kk[s] = nk;
  if (pass == 2) {
    P.kth[s] = prefix;
    P.ties[s] = nk;
  }
}

// -------------------------------------------------------------------------------- count
// Keys above and equal to the k-th, per candidate chunk (sorted) or per full-path tile.
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
  const uint32_t tg = block_sum<kThreads>(gt, s_tmp);
  const uint32_t te = block_sum<kThreads>(eq, s_tmp);
  if (threadIdx.x == 0) {
    *gt_out = tg;
    *eq_out = te;
  }
}

__device__ __forceinline__ void count_cand_chunk(const DevPlan& P, int64_t ch, uint32_t* s_tmp) {
  const int s = P.chunk_seg[ch];
  if (!has_candidates(P.mode[s])) return;
  const int64_t c = P.cand_cnt[s];
  const int64_t j0 = (ch - P.chunk_base[s]) * (int64_t)kChunk;
  if (j0 >= c) return;
  const int len = (int)min((int64_t)kChunk, c - j0);
  f4 x[kSlots];
  load_tile(P.sort_val + P.cand_base[s] + j0, len, x);
  count_block(x, len, P.kth[s], s_tmp, &P.chunk_gt[ch], &P.chunk_eq[ch]);
}

__device__ __forceinline__ void count_full_tiles(const DevPlan& P, const float* __restrict__ e,
                                                 int fb, uint32_t* s_tmp) {
  const uint32_t nf = *P.full_count;
  for (uint32_t li = 0; li < nf; ++li) {
    const int s = (int)P.full_list[li];
    const uint32_t kth = P.kth[s];
    for (int64_t t = P.tile_base[s] + fb; t < P.tile_base[s + 1]; t += kFullBlocks) {
      int64_t start;
      int len;
      tile_range(P, s, t, &start, &len);
      f4 x[kSlots];
      key_tile(P, e, start, len, x);
      count_block(x, len, kth, s_tmp, &P.tile_gt[t], &P.tile_eq[t]);
      uint32_t mx = 0;
      const int pb = slot_base();
#pragma unroll
      for (int v = 0; v < kSlots; ++v)
#pragma unroll
        for (int c = 0; c < 4; ++c)
          if (pb + v * 256 + c < len) mx = max(mx, mag_key(x[v][c]));
      mx = block_max<kThreads>(mx, s_tmp);
      if (threadIdx.x == 0) P.tile_max[t] = mx;
    }
  }
}

// Workgroups [0, n_chunk_blocks) count the active candidate chunks; the last kFullBlocks the
// tiles of the segments on the full path (one launch for both).
__global__ __launch_bounds__(kThreads) void k_count(DevPlan P, const float* __restrict__ e) {
  __shared__ uint32_t s_tmp[kWaves];
  if (blockIdx.x < (uint32_t)P.n_chunk_blocks) {
    const uint32_t na = *P.act_count;
    for (uint32_t i = blockIdx.x; i < na; i += (uint32_t)P.n_chunk_blocks)
      count_cand_chunk(P, P.act_chunk[i], s_tmp);
  } else {
    count_full_tiles(P, e, (int)(blockIdx.x - P.n_chunk_blocks), s_tmp);
  }
}

// --------------------------------------------------------------------------------- scan
// Per segment, over its chunks (candidates) or tiles (full path) in index order: ties
// before each item, then kept entries before each item (ties taken: the first `ties`).
__global__ __launch_bounds__(1024) void k_scan(DevPlan P, float* __restrict__ scales) {
  __shared__ uint32_t s_tmp[16];
  const int s = blockIdx.x;
  const uint32_t mode = P.mode[s];
  if (mode == kModeSkip) {
    if (scales && threadIdx.x == 0) scales[s] = 0.0f;  // fused int8: no kept values
    return;
  }
  const uint32_t r = P.ties[s];
  int64_t base, n;
  const uint32_t *GT, *EQ, *MX;
  uint32_t *EQB, *SELB;
  if (has_candidates(mode)) {
    base = P.chunk_base[s];
    n = ((int64_t)P.cand_cnt[s] + kChunk - 1) / kChunk;
    GT = P.chunk_gt; EQ = P.chunk_eq; EQB = P.chunk_eq_base; SELB = P.chunk_sel_base;
    MX = P.chunk_max;
  } else {
    base = P.tile_base[s];
    n = P.tile_base[s + 1] - base;
    GT = P.tile_gt; EQ = P.tile_eq; EQB = P.tile_eq_base; SELB = P.tile_sel_base;
    MX = P.tile_max;
  }
  uint32_t carry_eq = 0, carry_sel = 0, mx = 0;
  for (int64_t ib = 0; ib < n; ib += 1024) {
    const int64_t i = ib + threadIdx.x;
    const bool ok = i < n;
    const uint32_t gt = ok ? GT[base + i] : 0u, eq = ok ? EQ[base + i] : 0u;
    if (scales && ok) mx = max(mx, MX[base + i]);
    uint32_t tot_eq, tot_sel;
    const uint32_t eqb = carry_eq + block_excl_scan<1024>(eq, s_tmp, &tot_eq);
    const uint32_t take = eqb < r ? min(eq, r - eqb) : 0u;
    const uint32_t selb = carry_sel + block_excl_scan<1024>(gt + take, s_tmp, &tot_sel);
    if (ok) {
      EQB[base + i] = eqb;
      SELB[base + i] = selb;
    }
    carry_eq += tot_eq;
    carry_sel += tot_sel;
  }
  if (threadIdx.x == 0 && carry_sel != P.k[s]) atomicOr(P.err, 2u);
  if (scales) {  // fused int8: scale = fl(absmax / 127); the largest |acc| is always kept
    mx = block_max<1024>(mx, s_tmp);
    if (threadIdx.x == 0) scales[s] = __uint_as_float(mx) / 127.0f;
  }
}

// --------------------------------------------------------------------------------- emit
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
  const float* scales;       // fused int8: per-segment scales (written by k_scan)
  float scale;
  uint32_t seed_lo, seed_hi, step_lo;
  uint32_t* err;
  const float* vsrc;         // Random-k: kept values are read here (the tile holds keys)
  const float* rk_scale;     // Random-k without feedback: per-segment value scale, or null
  const float* vsrc_scale;   // Random-k reading g itself: the gradient scale, or null
  float vmul, gmul;
  __device__ float scales_of(int s) const { return scales[s]; }
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

__device__ __forceinline__ void emit_cand_chunk(const DevPlan& P, EmitOut o, int64_t ch,
                                                uint32_t* s_w) {
  const int s = P.chunk_seg[ch];
  if (!has_candidates(P.mode[s])) return;
  const int64_t c = P.cand_cnt[s];
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
  if (o.codes) o.scale = o.scales_of(s);
  if (o.rk_scale) o.vmul = o.rk_scale[s];
  if (o.vsrc_scale) o.gmul = o.vsrc_scale[s];
  emit_block(x, len, slot_idx, P.kth[s], P.ties[s], P.chunk_eq_base[ch], P.chunk_eq[ch],
             P.out_off[s] + P.chunk_sel_base[ch], P.out_off[s + 1], P.seg_off[s],
             (int32_t)(P.seg_off[s + 1] - P.seg_off[s]), s_w, o);
}

__device__ __forceinline__ void emit_full_tiles(const DevPlan& P, EmitOut o, int fb,
                                                uint32_t* s_w) {
  const uint32_t nf = *P.full_count;
  for (uint32_t li = 0; li < nf; ++li) {
    const int s = (int)P.full_list[li];
    const uint32_t kth = P.kth[s], r = P.ties[s];
    const int64_t s0 = P.seg_off[s];
    for (int64_t t = P.tile_base[s] + fb; t < P.tile_base[s + 1]; t += kFullBlocks) {
      int64_t start;
      int len;
      tile_range(P, s, t, &start, &len);
      f4 x[kSlots];
      key_tile(P, o.e, start, len, x);
      const int32_t lb = (int32_t)(start - s0) + slot_base();
      auto slot_idx = [&](int v) {
        const int32_t b0 = lb + v * 256;
        return i4{b0, b0 + 1, b0 + 2, b0 + 3};
      };
      if (o.codes) o.scale = o.scales_of(s);
      if (o.rk_scale) o.vmul = o.rk_scale[s];
      if (o.vsrc_scale) o.gmul = o.vsrc_scale[s];
      emit_block(x, len, slot_idx, kth, r, P.tile_eq_base[t], P.tile_eq[t],
                 P.out_off[s] + P.tile_sel_base[t], P.out_off[s + 1], s0,
                 (int32_t)(P.seg_off[s + 1] - s0), s_w, o);
    }
  }
}

// Workgroups [0, n_chunk_blocks) emit the active candidate chunks; the last kFullBlocks the
// tiles of the segments on the full path (one launch for both).
__global__ __launch_bounds__(kThreads) void k_emit(DevPlan P, EmitOut o) {
  __shared__ uint32_t s_w[kWaves];
  if (blockIdx.x < (uint32_t)P.n_chunk_blocks) {
    const uint32_t na = *P.act_count;
    for (uint32_t i = blockIdx.x; i < na; i += (uint32_t)P.n_chunk_blocks)
      emit_cand_chunk(P, o, P.act_chunk[i], s_w);
  } else {
    emit_full_tiles(P, o, (int)(blockIdx.x - P.n_chunk_blocks), s_w);
  }
}

// ---------------------------------------------------------------------------- cold start
// A plan's first call has no k-th key to start from.  Rather than capture nothing and
// re-capture every large segment from two extra passes over it, the call first forms acc on
// about 64 evenly spaced tiles of each such segment (exactly as the streaming pass will, but
// without storing it), histograms the first key digit, and sets the capture threshold
// GC_SAMPLE_MARGIN digits below the sample's estimate of the k-th key.  A wrong estimate only costs the usual
// re-capture: the candidates are checked for completeness as on every call.
__global__ __launch_bounds__(kThreads) void k_sample_zero(DevPlan P) {
  const int s = blockIdx.x;
  if (P.sample_elems[s] == 0) return;
  uint32_t* h = P.hist + (size_t)s * 3 * kHistBins;
  for (int i = threadIdx.x; i < kHistBins; i += kThreads) h[i] = 0;
}

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
  hist_flush(h, P.hist + (size_t)s * 3 * kHistBins);
}

// Per sampled segment still without an estimate: the first-digit bucket d that holds the
// sample's ceil(k * sample / n)-th largest key; the threshold is the floor of bucket
// d - GC_SAMPLE_MARGIN.
__global__ __launch_bounds__(kThreads) void k_sample_decide(DevPlan P) {
  __shared__ uint32_t s_tmp[kWaves];
  __shared__ uint32_t s_out[3];
  const int s = blockIdx.x;
  const int64_t ns = P.sample_elems[s];
  if (ns == 0 || P.thr[s] != kNoCapture) return;
  const int64_t n = P.seg_off[s + 1] - P.seg_off[s];
  const int64_t k = P.k[s];
  const uint32_t kk = (uint32_t)max((int64_t)1, (k * ns + n - 1) / n);
  uint32_t d, above, bin;
  const bool ok = find_digit(P.hist + (size_t)s * 3 * kHistBins, kk, s_tmp, s_out, &d, &above,
                             &bin);
  if (threadIdx.x == 0 && ok)
    P.thr[s] = d > (uint32_t)GC_SAMPLE_MARGIN ? (d - (uint32_t)GC_SAMPLE_MARGIN) << 20 : 0u;
}

// ----------------------------------------------------------------------------- finalize
// Threshold for the next call: beta * |kth|, where the margin beta follows the last calls:
// lowered after too few candidates, raised after an overflow or far more than needed, and
// kept in [0.25, GC_BETA_MAX]; a cap near 1 suits a residual that still grows, whose next
// k-th key lies above the last one.
// Segments that capture everything (small) or nothing (k = 0) keep their setting.
__global__ __launch_bounds__(kThreads) void k_finalize(DevPlan P) {
  const int s = blockIdx.x * kThreads + threadIdx.x;
  if (s >= P.n_seg) return;
  const uint32_t init = P.thr_init[s], mode = P.mode[s];
  uint32_t next = init;
  if (init == kNoCapture && mode != kModeSkip && !(P.flags & (kFlagForceFull | kFlagNoEstimate))) {
    float b = P.beta[s];
    const uint32_t why = P.why[s];
    if (why == kWhyMiss) {
      b = fmaxf(b * 0.85f, 0.25f);
    } else if (why == kWhyOverflow) {
      b = fminf(b * 1.05f, GC_BETA_MAX);
    } else if (mode == kModeCand) {
      const float rho = (float)P.cand_cnt[s] / (float)P.k[s];
      if (rho > GC_RHO_HIGH) b = fminf(b * 1.03f, GC_BETA_MAX);
      else if (rho < GC_RHO_LOW) b = fmaxf(b * 0.97f, 0.25f);
    }
    P.beta[s] = b;
    next = mag_key(b * __uint_as_float(P.kth[s]));
  }
  P.thr[s] = next;
}

// Threshold calls: the capture floor for the next call, by the rule of k_finalize applied to
// this call's k (so it tracks the k-th largest kept key while the cap binds and falls below
// key(|tau|), where it has no effect, while it does not).
__global__ __launch_bounds__(kThreads) void k_finalize_thr(DevPlan P) {
  const int s = blockIdx.x * kThreads + threadIdx.x;
  if (s >= P.n_seg) return;
  const uint32_t mode = P.mode[s];
  if (P.thr_init[s] != kNoCapture || mode == kModeSkip ||
      (P.flags & (kFlagForceFull | kFlagNoEstimate)))
    return;   // small segments capture everything; k = 0 keeps its floor
  float b = P.beta_est[s];
  const uint32_t why = P.why[s];
  if (why == kWhyMiss) {
    b = fmaxf(b * 0.85f, 0.25f);
  } else if (why == kWhyOverflow) {
    b = fminf(b * 1.05f, GC_BETA_MAX);
  } else if (mode == kModeCand) {
    const float rho = (float)P.cand_cnt[s] / (float)P.k_call[s];
    if (rho > GC_RHO_HIGH) b = fminf(b * 1.03f, GC_BETA_MAX);
    else if (rho < GC_RHO_LOW) b = fmaxf(b * 0.97f, 0.25f);
  }
  P.beta_est[s] = b;
  P.thr_est[s] = mag_key(b * __uint_as_float(P.kth[s]));
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
  capture_tile(P, s, t, start, len, key, thr, s_w, &s_base);
}

// Random-k without error feedback or momentum reads nothing in its pass: it only draws keys
// and captures the ones at or above the threshold, as k_randk_capture does, with the same
// runs and order.  With no memory stream to hide behind, the workgroup-wide ranks and barriers
// of the tile layout dominate, so here one wave owns a whole tile: slot v (0 .. kTile/256 - 1)
// of lane l holds the 4 elements from v * 256 + l * 4 (index order is slot, lane, element).
// The wave draws its keys slot by slot, ranks the flagged ones with ballots as it goes and
// stages the first kRkStage of them (key, tile offset) in its own LDS rows; then it reserves
// the tile's run with one atomic and copies the staged entries out.  Entries past the staging
// rows (dense segments) are drawn again from the per-slot flags.  No barrier anywhere.
constexpr int kRkWaves = 4;
constexpr int kRkSlots = kTile / 256;
constexpr int kRkStage = 256;
static_assert(kRkSlots % 8 == 0, "a tile must hold whole words of eight 256-element slots");

template <bool kAligned>
__device__ __forceinline__ void rk_tile(const DevPlan& P, int64_t t, int64_t start, int len,
                                        int s, uint32_t thr, int lane, uint32_t* sk,
                                        int32_t* si) {
  uint32_t pk[kRkSlots / 8];   // flags, one nibble per slot (the word loop is unrolled)
  uint32_t cnt = 0;            // wave-uniform: flagged entries so far
#pragma unroll
  for (int wi = 0; wi < kRkSlots / 8; ++wi) {
    uint32_t word = 0;
    for (int j = 0; j < 8; ++j) {
      const int p0 = (wi * 8 + j) * 256 + lane * 4;
      uint32_t k[4];
      rand_key4<kAligned>(P, start + p0, k);
      uint32_t nib = 0;
#pragma unroll
      for (int c = 0; c < 4; ++c) nib |= (p0 + c < len && k[c] >= thr) ? (1u << c) : 0u;
      word |= nib << (4 * j);
      if (!__ballot(nib != 0)) continue;   // uniform
      const uint64_t m0 = __ballot(nib & 1u), m1 = __ballot(nib & 2u);
      const uint64_t m2 = __ballot(nib & 4u), m3 = __ballot(nib & 8u);
      uint32_t r = cnt + lanes_below(m0) + lanes_below(m1) + lanes_below(m2) + lanes_below(m3);
      cnt += __popcll(m0) + __popcll(m1) + __popcll(m2) + __popcll(m3);
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if ((nib >> c) & 1u) {
          if (r < (uint32_t)kRkStage) {
            sk[r] = k[c];
            si[r] = p0 + c;
          }
          ++r;
        }
    }
    pk[wi] = word;
  }
  uint32_t base = 0;
  if (lane == 0) {
    base = cnt ? atomicAdd(&P.cand_cnt[s], cnt) : 0u;
    P.run_off[t] = base;
    P.run_cnt[t] = cnt;
  }
  if (cnt == 0) return;   // uniform
  base = __shfl(base, 0, 64);
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
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t t = (int64_t)blockIdx.x * kRkWaves + w;
  if (t >= P.n_tiles) return;   // wave-uniform
  const int4 desc = P.tile_desc[t];
  const int64_t start = (int64_t)(((uint64_t)(uint32_t)desc.y << 32) | (uint32_t)desc.x);
  const int len = desc.z, s = desc.w;
  const uint32_t thr = P.thr[s];
  if (thr == kNoCapture) return;   // this segment takes the exact fallback
  if ((start & 3) == 0)   // wave-uniform: every lane's four elements share one Philox block
    rk_tile<true>(P, t, start, len, s, thr, lane, s_key[w], s_idx[w]);
  else
    rk_tile<false>(P, t, start, len, s, thr, lane, s_key[w], s_idx[w]);
}

// Threshold call: slots past the segment's kept entries get value +0 and index -1.
__global__ __launch_bounds__(kThreads) void k_pad_out(OutPlan O, const uint32_t* __restrict__ k_call,
                                                      float* __restrict__ vals,
                                                      int32_t* __restrict__ idx) {
  const int64_t ch = blockIdx.x;
  const int s = O.out_chunk_seg[ch];
  const int64_t j0 = O.out_off[s] + (ch - O.out_chunk_base[s]) * (int64_t)kOutChunk;
  const int64_t j1 = min(j0 + kOutChunk, O.out_off[s + 1]);
  const int64_t keep_end = O.out_off[s] + k_call[s];
  for (int64_t j = max(j0, keep_end) + threadIdx.x; j < j1; j += kThreads) {
    vals[j] = 0.0f;
    idx[j] = -1;
  }
}

// Everything after the streaming pass: select (candidates, re-capture or the exact full
// path), ordered count/scan, emit.  e holds acc (magnitude keys); scales: fused int8 or null.
void select_emit(const DevPlan& P, const float* e, const EmitOut& o, float* scales,
                 hipStream_t st) {
  k_select_init<<<P.n_seg, kThreads, 0, st>>>(P);
  k_recap_hist<<<kFullBlocks, kThreads, 0, st>>>(P, e);
  k_recap_decide<<<P.n_seg, kThreads, 0, st>>>(P);
  k_recapture<<<kFullBlocks, kThreads, 0, st>>>(P, e);
  k_runs<<<P.n_seg, 1024, 0, st>>>(P);
  if (P.n_chunk_blocks > 0) k_scatter<<<(unsigned)P.n_chunk_blocks, kThreads, 0, st>>>(P);
  k_find<<<P.n_seg, kThreads, 0, st>>>(P, 0);
  const unsigned mixed = (unsigned)(P.n_chunk_blocks + kFullBlocks);
  for (int pass = 1; pass < 3; ++pass) {
    k_hist<<<mixed, kThreads, 0, st>>>(P, e, pass);
    k_find<<<P.n_seg, kThreads, 0, st>>>(P, pass);
  }
  k_count<<<mixed, kThreads, 0, st>>>(P, e);
  k_scan<<<P.n_seg, 1024, 0, st>>>(P, scales);
  k_emit<<<mixed, kThreads, 0, st>>>(P, o);
}

}  // namespace

hipError_t launch_compress(const DevPlan& P, const float* g, float* e, float* u, float m,
                           float* out_vals, int32_t* out_idx, const Int8Args& q8, bool cold,
                           hipStream_t st, hipEvent_t ev_begin, hipEvent_t ev_end) {
  if (P.n_seg == 0) return hipSuccess;
  k_prep<<<blocks_for(P.n_seg, kThreads), kThreads, 0, st>>>(P);
  if (cold && P.n_sample > 0) {
    k_sample_zero<<<P.n_seg, kThreads, 0, st>>>(P);
    if (u)
      k_sample_hist<true><<<(unsigned)P.n_sample, kThreads, 0, st>>>(P, g, e, u, m);
    else
      k_sample_hist<false><<<(unsigned)P.n_sample, kThreads, 0, st>>>(P, g, e, nullptr, m);
    k_sample_decide<<<P.n_seg, kThreads, 0, st>>>(P);
  }
  if (ev_begin) (void)hipEventRecord(ev_begin, st);
  if (P.n_tiles > 0) {
    const unsigned nt = (unsigned)P.n_tiles;
    if (P.gscale) {
      if (u) k_ef_capture<true, false, true><<<nt, kThreads, 0, st>>>(P, g, e, u, m);
      else k_ef_capture<false, false, true><<<nt, kThreads, 0, st>>>(P, g, e, nullptr, m);
    } else {
      if (u) k_ef_capture<true><<<nt, kThreads, 0, st>>>(P, g, e, u, m);
      else k_ef_capture<false><<<nt, kThreads, 0, st>>>(P, g, e, nullptr, m);
    }
  }
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
  select_emit(P, e, o, q8.enabled ? q8.scales : nullptr, st);
  k_finalize<<<blocks_for(P.n_seg, kThreads), kThreads, 0, st>>>(P);
  return hipGetLastError();
}

hipError_t launch_threshold(const DevPlan& P, const OutPlan& O, const float* g, float* e,
                            float* u, float m, const float* tau, float* out_vals,
                            int32_t* out_idx, int32_t* out_count, hipStream_t st,
                            hipEvent_t ev_begin, hipEvent_t ev_end) {
  if (P.n_seg == 0) return hipSuccess;
  DevPlan Q = P;
  Q.k = P.k_call;
  Q.thr = P.thr_call;
  Q.keys = kKeysMagnitude;
  k_prep_call<<<blocks_for(P.n_seg, kThreads), kThreads, 0, st>>>(P, tau);
  if (ev_begin) (void)hipEventRecord(ev_begin, st);
  if (P.n_tiles > 0) {
    const unsigned nt = (unsigned)P.n_tiles;
    if (P.gscale) {
      if (u) k_ef_capture<true, true, true><<<nt, kThreads, 0, st>>>(Q, g, e, u, m);
      else k_ef_capture<false, true, true><<<nt, kThreads, 0, st>>>(Q, g, e, nullptr, m);
    } else {
      if (u) k_ef_capture<true, true><<<nt, kThreads, 0, st>>>(Q, g, e, u, m);
      else k_ef_capture<false, true><<<nt, kThreads, 0, st>>>(Q, g, e, nullptr, m);
    }
  }
  if (ev_end) (void)hipEventRecord(ev_end, st);
  k_thresh_k<<<blocks_for(P.n_seg, kThreads), kThreads, 0, st>>>(P, out_count);
  EmitOut o{};
  o.e = e;
  o.u = (u && (P.flags & kFlagMomentumMask)) ? u : nullptr;
  o.vals = out_vals;
  o.idx = out_idx;
  o.err = P.err;
  select_emit(Q, e, o, nullptr, st);
  if (O.n_out_chunks > 0)
    k_pad_out<<<(unsigned)O.n_out_chunks, kThreads, 0, st>>>(O, P.k_call, out_vals, out_idx);
  k_finalize_thr<<<blocks_for(P.n_seg, kThreads), kThreads, 0, st>>>(P);
  return hipGetLastError();
}

hipError_t launch_randk(const DevPlan& P, const float* g, float* e, float* u, float m,
                        uint64_t seed, uint64_t step, float* out_vals, int32_t* out_idx,
                        hipStream_t st, hipEvent_t ev_begin, hipEvent_t ev_end) {
  if (P.n_seg == 0) return hipSuccess;
  DevPlan Q = P;
  Q.k = P.k_call;
  Q.thr = P.thr_call;
  Q.keys = kKeysRandom;
  Q.seed_lo = (uint32_t)seed;
  Q.seed_hi = (uint32_t)(seed >> 32);
  Q.step_lo = (uint32_t)step;
  k_prep_call<<<blocks_for(P.n_seg, kThreads), kThreads, 0, st>>>(P, nullptr);
  if (ev_begin) (void)hipEventRecord(ev_begin, st);
  if (P.n_tiles > 0) {
    const unsigned nt = (unsigned)P.n_tiles;
    if (P.gscale) {
      if (e && u) k_randk_capture<true, true, true><<<nt, kThreads, 0, st>>>(Q, g, e, u, m);
      else if (e) k_randk_capture<false, true, true><<<nt, kThreads, 0, st>>>(Q, g, e, nullptr, m);
      else if (u) k_randk_capture<true, false, true><<<nt, kThreads, 0, st>>>(Q, g, nullptr, u, m);
      // neither: the capture reads no g (the emit applies the scale to the gathered values)
      else k_randk_keys<<<blocks_for(P.n_tiles, kRkWaves), kRkWaves * 64, 0, st>>>(Q);
    } else {
      if (e && u) k_randk_capture<true, true><<<nt, kThreads, 0, st>>>(Q, g, e, u, m);
      else if (e) k_randk_capture<false, true><<<nt, kThreads, 0, st>>>(Q, g, e, nullptr, m);
      else if (u) k_randk_capture<true, false><<<nt, kThreads, 0, st>>>(Q, g, nullptr, u, m);
      else k_randk_keys<<<blocks_for(P.n_tiles, kRkWaves), kRkWaves * 64, 0, st>>>(Q);
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
  select_emit(Q, e, o, nullptr, st);
  return hipGetLastError();
}

hipError_t launch_reset(const DevPlan& P, hipStream_t st) {
  if (P.n_seg == 0) return hipSuccess;
  k_reset<<<blocks_for(P.n_seg, kThreads), kThreads, 0, st>>>(P);
  return hipGetLastError();
}

}  // namespace gc
