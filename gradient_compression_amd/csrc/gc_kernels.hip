// gc_kernels.hip -- gfx950 kernels of the error-feedback gradient compressors.
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
// magnitudes.  The 1-bit sign and QSGD codecs are two streaming passes around a per-segment
// scale; decompression and the receiver-side sum are scatters.
//
// The method is the Top-K with error feedback of "Communication Optimization > Gradient
// Compression" (Top-K section equations); momentum correction per the "Gradient
// Sparsification" glossary; the int8 stage per the "Gradient Compression" glossary
// (Top-k then 8-bit) with stochastic rounding (QSGD paragraph) and one scale per layer.
#include "gc_internal.h"

#pragma clang fp contract(off)

namespace gc {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef int i4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t mag_key(float x) { return __float_as_uint(x) & 0x7FFFFFFFu; }

// Factor on the gradient of segment s: x = fl(g * f) in place of g when the plan carries a
// per-segment gradient scale (clipping folded into the load), else 1 (fl(g * 1) = g exactly).
__device__ __forceinline__ float grad_scale(const DevPlan& P, int s) {
  return P.gscale ? P.gscale[s] : 1.0f;
}

// Number of set bits of m at lanes below this lane.
__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }
// First element (tile-relative) of this lane's slot 0.
__device__ __forceinline__ int slot_base() { return wave_id() * kWaveSpan + lane_id() * 4; }

// Philox4x32-10 (Salmon et al., SC'11), word 0 of the output block.
__device__ __forceinline__ uint32_t philox_word0(uint32_t c0, uint32_t c1, uint32_t c2,
                                                 uint32_t c3, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int round = 0; round < 10; ++round) {
    // one 32x32->64 product per multiplier (a single v_mad_u64_u32 gives both halves)
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0, p1 = (uint64_t)0xCD9E8D57u * c2;
    const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    const uint32_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return c0;
}

// Philox4x32-10 (Salmon et al., SC'11), all four words of the output block.
__device__ __forceinline__ void philox4(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                        uint32_t k0, uint32_t k1, uint32_t (&out)[4]) {
#pragma unroll
  for (int round = 0; round < 10; ++round) {
    // one 32x32->64 product per multiplier (a single v_mad_u64_u32 gives both halves)
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0, p1 = (uint64_t)0xCD9E8D57u * c2;
    const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    const uint32_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  out[0] = c0;
  out[1] = c1;
  out[2] = c2;
  out[3] = c3;
}

// Stochastic level from a given 24-bit draw: a = min(|v|/scale, limit), level floor(a) or
// floor(a) + 1 when u24 < frac(a) * 2^24; returns sign(v) * level, *deq = fl(code * scale).
__device__ __forceinline__ int sr_code_u24(float v, float scale, float limit, uint32_t u24,
                                           float* deq) {
  int q = 0;
  if (scale != 0.0f) {
    float a = fabsf(v) / scale;
    if (a > limit) a = limit;
    const float f = floorf(a);
    const float frac = a - f;
    q = (int)f + (((float)u24 < frac * 16777216.0f) ? 1 : 0);
  }
  const int code = signbit(v) ? -q : q;
  *deq = (float)code * scale;
  return code;
}

// Stochastic level of v (global index gi) at quantisation step `scale`: a = min(|v|/scale,
// limit), level floor(a) or floor(a) + 1 with probability frac(a) (top 24 bits of Philox
// word 0 at counter (gi lo, gi hi, step lo, tag)); returns sign(v) * level and writes the
// dequantised value fl(code * scale) to *deq.  scale == 0 gives code 0.
__device__ __forceinline__ int sr_code(float v, float scale, float limit, int64_t gi,
                                       uint32_t seed_lo, uint32_t seed_hi, uint32_t step_lo,
                                       uint32_t tag, float* deq) {
  int q = 0;
  if (scale != 0.0f) {
    float a = fabsf(v) / scale;
    if (a > limit) a = limit;
    const float f = floorf(a);
    const float frac = a - f;
    const uint32_t u24 = philox_word0((uint32_t)gi, (uint32_t)((uint64_t)gi >> 32), step_lo,
                                      tag, seed_lo, seed_hi) >> 8;
    q = (int)f + (((float)u24 < frac * 16777216.0f) ? 1 : 0);
  }
  const int code = signbit(v) ? -q : q;
  *deq = (float)code * scale;
  return code;
}

// The int8 stage of a kept value: 127 levels of fl(absmax / 127), counter tag 0x51.
__device__ __forceinline__ int quant_code(float v, float scale, int64_t gi, uint32_t seed_lo,
                                          uint32_t seed_hi, uint32_t step_lo, float* deq) {
  return sr_code(v, scale, 127.0f, gi, seed_lo, seed_hi, step_lo, 0x51u, deq);
}

// Exclusive scan of one uint32 per thread over a block of NT threads; *total gets the sum.
// s_tmp: __shared__ uint32_t[NT / 64].  Contains barriers: call from every thread.
template <int NT>
__device__ uint32_t block_excl_scan(uint32_t v, uint32_t* s_tmp, uint32_t* total) {
  const int lane = lane_id(), w = wave_id();
  uint32_t x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63) s_tmp[w] = x;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) {
    const uint32_t t = s_tmp[i];
    before += (i < w) ? t : 0u;
    tot += t;
  }
  __syncthreads();
  *total = tot;
  return before + x - v;
}

// Largest value over a block of NT threads (valid in every thread).  s_tmp: [NT / 64].
template <int NT>
__device__ uint32_t block_max(uint32_t v, uint32_t* s_tmp) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v = max(v, (uint32_t)__shfl_xor(v, d, 64));
  if (lane_id() == 0) s_tmp[wave_id()] = v;
  __syncthreads();
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) m = max(m, s_tmp[i]);
  __syncthreads();
  return m;
}

// Sum over a block of NT threads (result valid in every thread).
template <int NT>
__device__ uint32_t block_sum(uint32_t v, uint32_t* s_tmp) {
  uint32_t tot;
  block_excl_scan<NT>(v, s_tmp, &tot);
  return tot;
}

// Ordered ranks of the flagged elements of a tile laid out as (wave, slot, lane, element).
// bits[v] holds the 4 flags of this lane's slot v.  On return woff[v] is the number of flagged
// elements of the tile that come before this lane's slot v; the return value is the tile's
// total.  Element c of slot v then has rank woff[v] + popcount(bits[v] & ((1 << c) - 1)).
// s_w: __shared__ uint32_t[kWaves].  Contains barriers: call from every thread.
__device__ uint32_t tile_rank(const uint32_t (&bits)[kSlots], uint32_t (&woff)[kSlots],
                              uint32_t* s_w) {
  uint32_t any = 0;
#pragma unroll
  for (int v = 0; v < kSlots; ++v) any |= bits[v];
  uint32_t run = 0;
  if (__ballot(any != 0)) {
#pragma unroll
    for (int v = 0; v < kSlots; ++v) {
      const uint32_t b = bits[v];
      const uint64_t m0 = __ballot(b & 1u), m1 = __ballot(b & 2u);
      const uint64_t m2 = __ballot(b & 4u), m3 = __ballot(b & 8u);
      woff[v] = run + lanes_below(m0) + lanes_below(m1) + lanes_below(m2) + lanes_below(m3);
      run += __popcll(m0) + __popcll(m1) + __popcll(m2) + __popcll(m3);
    }
  } else {
#pragma unroll
    for (int v = 0; v < kSlots; ++v) woff[v] = 0;
  }
  if (lane_id() == 0) s_w[wave_id()] = run;
  __syncthreads();
  uint32_t before = 0, total = 0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) {
    const uint32_t x = s_w[i];
    before += (i < wave_id()) ? x : 0u;
    total += x;
  }
  __syncthreads();
#pragma unroll
  for (int v = 0; v < kSlots; ++v) woff[v] += before;
  return total;
}

// Load the len (<= kTile) elements at base into the tile layout; lanes past len get 0.
// The vector path needs base 16-byte aligned and a whole tile.
template <typename V, typename S>
__device__ __forceinline__ void load_tile(const S* __restrict__ base, int len, V (&x)[kSlots]) {
  const int pb = slot_base();
  if (len == kTile && ((reinterpret_cast<uintptr_t>(base) & 15) == 0)) {
    const V* b4 = reinterpret_cast<const V*>(base);
#pragma unroll
    for (int v = 0; v < kSlots; ++v) x[v] = b4[(pb + v * 256) >> 2];
  } else {
#pragma unroll
    for (int v = 0; v < kSlots; ++v)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int p = pb + v * 256 + c;
        x[v][c] = p < len ? base[p] : S(0);
      }
  }
}

// Random-k keys of the len (<= kTile) elements from global index start, in the tile layout,
// as float bit patterns: word (gi % 4) of the Philox4x32-10 block keyed (seed lo, seed hi) at
// counter (gi / 4 lo, gi / 4 hi, step lo, 0x53), shifted right by one (31 bits).  A lane's
// four elements share one block when start is a multiple of 4.  Lanes past len get key 0.
__device__ __forceinline__ void rand_key_tile(const DevPlan& P, int64_t start, int len,
                                              f4 (&x)[kSlots]) {
  const int pb = slot_base();
#pragma unroll
  for (int v = 0; v < kSlots; ++v) {
    const int64_t g0 = start + pb + v * 256;
    const uint64_t b0 = (uint64_t)g0 >> 2;
    uint32_t w[4], w2[4] = {0u, 0u, 0u, 0u};
    philox4((uint32_t)b0, (uint32_t)(b0 >> 32), P.step_lo, 0x53u, P.seed_lo, P.seed_hi, w);
    if (g0 & 3)
      philox4((uint32_t)(b0 + 1), (uint32_t)((b0 + 1) >> 32), P.step_lo, 0x53u, P.seed_lo,
              P.seed_hi, w2);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int j = (int)(g0 & 3) + c;   // position of element c from the first block
      const uint32_t word = j < 4 ? w[j] : w2[j - 4];
      x[v][c] = pb + v * 256 + c < len ? __uint_as_float(word >> 1) : 0.0f;
    }
  }
}

// What the select ranks for the tile at start: acc read back from e (its magnitude key), or
// the elements' Random-k keys.
__device__ __forceinline__ void key_tile(const DevPlan& P, const float* __restrict__ e,
                                         int64_t start, int len, f4 (&x)[kSlots]) {
  if (P.keys == kKeysRandom)
    rand_key_tile(P, start, len, x);
  else
    load_tile(e + start, len, x);
}

// ------------------------------------------------------------------------------ prep
__global__ __launch_bounds__(kThreads) void k_prep(DevPlan P) {
  const int s = blockIdx.x * kThreads + threadIdx.x;
  if (s < P.n_seg) P.cand_cnt[s] = 0;
  if (s == 0) {
    *P.full_count = 0;
    *P.recap_count = 0;
    *P.err = 0;
  }
}

__global__ __launch_bounds__(kThreads) void k_reset(DevPlan P) {
  const int s = blockIdx.x * kThreads + threadIdx.x;
  if (s < P.n_seg) {
    P.thr[s] = P.thr_init[s];
    P.thr_est[s] = kNoCapture;
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
__global__ __launch_bounds__(1024) void k_runs(DevPlan P) {
  __shared__ uint32_t s_tmp[16];
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
}

// ------------------------------------------------------------------------------ scatter
// Candidates into ascending index order (tile t's run goes to run_dst[t]); on the estimate
// path, also the first-digit histogram of the candidates.
__global__ __launch_bounds__(kThreads) void k_scatter(DevPlan P) {
  __shared__ uint32_t h[kHistBins];
  const int64_t ch = blockIdx.x;
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
  __shared__ uint32_t s_m[kWaves];
  mx = block_max<kThreads>(mx, s_m);
  if (threadIdx.x == 0) P.chunk_max[ch] = mx;
  if (do_hist) {
    __syncthreads();
    hist_flush(h, P.hist + (size_t)s * 3 * kHistBins);
  }
}

// --------------------------------------------------------------------------------- hist
// Passes 1 and 2.  Workgroups [0, n_chunks) histogram sorted candidate chunks; the last
// kFullBlocks histogram the tiles of the segments on the full path.
__global__ __launch_bounds__(kThreads) void k_hist(DevPlan P, const float* __restrict__ e,
                                                   int pass) {
  __shared__ uint32_t h[kHistBins];
  if (blockIdx.x < P.n_chunks) {
    const int64_t ch = blockIdx.x;
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
    return;
  }
  hist_listed_tiles(P, e, P.full_list, *P.full_count, kModeFull, pass,
                    blockIdx.x - (int)P.n_chunks, h);
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

__global__ __launch_bounds__(kThreads) void k_count_cand(DevPlan P) {
  __shared__ uint32_t s_tmp[kWaves];
  const int64_t ch = blockIdx.x;
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

__global__ __launch_bounds__(kThreads) void k_count_full(DevPlan P, const float* __restrict__ e) {
  __shared__ uint32_t s_tmp[kWaves];
  const uint32_t nf = *P.full_count;
  for (uint32_t li = 0; li < nf; ++li) {
    const int s = (int)P.full_list[li];
    const uint32_t kth = P.kth[s];
    for (int64_t t = P.tile_base[s] + blockIdx.x; t < P.tile_base[s + 1]; t += kFullBlocks) {
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

__global__ __launch_bounds__(kThreads) void k_emit_cand(DevPlan P, EmitOut o) {
  __shared__ uint32_t s_w[kWaves];
  const int64_t ch = blockIdx.x;
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

__global__ __launch_bounds__(kThreads) void k_emit_full(DevPlan P, EmitOut o) {
  __shared__ uint32_t s_w[kWaves];
  const uint32_t nf = *P.full_count;
  for (uint32_t li = 0; li < nf; ++li) {
    const int s = (int)P.full_list[li];
    const uint32_t kth = P.kth[s], r = P.ties[s];
    const int64_t s0 = P.seg_off[s];
    for (int64_t t = P.tile_base[s] + blockIdx.x; t < P.tile_base[s + 1]; t += kFullBlocks) {
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

// ----------------------------------------------------------------------------- finalize
// Threshold for the next call: beta * |kth|, where the margin beta follows the last calls:
// lowered after too few candidates, raised after an overflow or far more than needed.  beta
// may exceed 1: while the residual still grows, the next k-th key lies above the last one.
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

// ------------------------------------------------------------------------ 1-bit sign
// 1-bit sign compression with error feedback ("Communication Optimization > Gradient
// Compression", 1-bit SGD section: Q(g) = sign(g) * ||g||_1 / d, one scale per layer; error
// feedback as for top-K).  Pass 1 takes each tile's sum of |acc| in double (with momentum it
// also stores u and acc = e + u; without, it only reads and pass 2 forms acc = e + g again);
// the scale is fl32(S / n) per segment; pass 2 writes the sign bits (bit i of word i/32,
// 1 = negative) and the residual e = fl(acc - sign * scale).

// Load the tile of g (and u), form acc (momentum first, x = fl(g * gf)), store acc into e
// (and u).
template <bool kMomentum>
__device__ __forceinline__ void ef_add_tile(const float* __restrict__ g, float gf,
                                            float* __restrict__ e, float* __restrict__ u,
                                            float m, int64_t start, int len,
                                            f4 (&acc)[kSlots]) {
  const int pb = slot_base();
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
}

// load_tile for a streaming pass: the full-tile loads are non-temporal.
__device__ __forceinline__ void load_tile_nt(const float* __restrict__ base, int len,
                                             f4 (&x)[kSlots]) {
  const int pb = slot_base();
  if (len == kTile && ((reinterpret_cast<uintptr_t>(base) & 15) == 0)) {
    const f4* b4 = reinterpret_cast<const f4*>(base);
#pragma unroll
    for (int v = 0; v < kSlots; ++v) x[v] = __builtin_nontemporal_load(b4 + ((pb + v * 256) >> 2));
  } else {
    load_tile(base, len, x);
  }
}

// acc = fl(e + fl(g * gf)) over one tile without storing it (lanes past len get 0): the two-pass
// codecs without momentum form acc in both passes, so their first pass only reads.
__device__ __forceinline__ void acc_tile(const float* __restrict__ g, float gf,
                                         const float* __restrict__ e, int64_t start, int len,
                                         f4 (&acc)[kSlots]) {
  const int pb = slot_base();
  if (len == kTile && (start & 3) == 0) {
    const f4* g4 = reinterpret_cast<const f4*>(g + start);
    const f4* e4 = reinterpret_cast<const f4*>(e + start);
    f4 gv[kSlots];
#pragma unroll
    for (int v = 0; v < kSlots; ++v) {
      const int q = (pb + v * 256) >> 2;
      gv[v] = GC_NT_LOAD_G ? __builtin_nontemporal_load(g4 + q) : g4[q];
      acc[v] = GC_NT_LOAD_E ? __builtin_nontemporal_load(e4 + q) : e4[q];
    }
#pragma unroll
    for (int v = 0; v < kSlots; ++v) acc[v] = acc[v] + gv[v] * gf;
  } else {
#pragma unroll
    for (int v = 0; v < kSlots; ++v)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int p = pb + v * 256 + c;
        acc[v][c] = p < len ? e[start + p] + g[start + p] * gf : 0.0f;
      }
  }
}

// Pass 1: per-tile sum of |acc|.  With momentum acc (and u) is stored for pass 2; without,
// nothing is written and pass 2 forms acc again from g and e.
template <bool kMomentum>
__global__ __launch_bounds__(kThreads) void k_sign_pass1(DevPlan P, const float* __restrict__ g,
                                                        float* __restrict__ e,
                                                        float* __restrict__ u, float m) {
  __shared__ double s_d[kWaves];
  const int64_t t = blockIdx.x;
  const int4 desc = P.tile_desc[t];
  const int64_t start = (int64_t)(((uint64_t)(uint32_t)desc.y << 32) | (uint32_t)desc.x);
  const int len = desc.z;
  const float gf = grad_scale(P, desc.w);
  f4 acc[kSlots];
  if (kMomentum)
    ef_add_tile<true>(g, gf, e, u, m, start, len, acc);
  else
    acc_tile(g, gf, e, start, len, acc);
  double l1 = 0.0;   // lanes past len hold 0
#pragma unroll
  for (int v = 0; v < kSlots; ++v)
#pragma unroll
    for (int c = 0; c < 4; ++c) l1 += fabs((double)acc[v][c]);
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) l1 += __shfl_xor(l1, d, 64);
  if (lane_id() == 0) s_d[wave_id()] = l1;
  __syncthreads();
  if (threadIdx.x == 0) {
    double sum = 0.0;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) sum += s_d[i];
    P.tile_l1[t] = sum;
  }
}

// Per segment: scale = fl32(S / n), S = the tiles' sums (a fixed tree order).
__global__ __launch_bounds__(1024) void k_sign_scale(DevPlan P, float* __restrict__ scales) {
  __shared__ double s_d[16];
  const int s = blockIdx.x;
  const int64_t t0 = P.tile_base[s], t1 = P.tile_base[s + 1];
  double sum = 0.0;
  for (int64_t t = t0 + threadIdx.x; t < t1; t += 1024) sum += P.tile_l1[t];
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) sum += __shfl_xor(sum, d, 64);
  if (lane_id() == 0) s_d[wave_id()] = sum;
  __syncthreads();
  if (threadIdx.x == 0) {
    double tot = 0.0;
    for (int i = 0; i < 16; ++i) tot += s_d[i];
    const int64_t n = P.seg_off[s + 1] - P.seg_off[s];
    scales[s] = n > 0 ? (float)(tot / (double)n) : 0.0f;
  }
}

// Sign bits of one tile-shaped block: lane l of slot v covers 4 elements of the 32-element
// word (w*kSlots + v)*8 + l/8 (tile-relative); its nibble lands at bit 4*(l%8).
// kRecompute: acc = e + g formed here (no momentum); else acc was stored into e by pass 1.
template <bool kRecompute>
__global__ __launch_bounds__(kThreads) void k_sign_pass2(DevPlan P, const float* __restrict__ g,
                                                        float* __restrict__ e,
                                                        uint32_t* __restrict__ bits,
                                                        const float* __restrict__ scales) {
  const int64_t t = blockIdx.x;
  const int4 desc = P.tile_desc[t];
  const int64_t start = (int64_t)(((uint64_t)(uint32_t)desc.y << 32) | (uint32_t)desc.x);
  const int len = desc.z, s = desc.w;
  const float scale = scales[s];
  const int pb = slot_base(), lane = lane_id();
  f4 acc[kSlots];
  if (kRecompute)
    acc_tile(g, grad_scale(P, s), e, start, len, acc);
  else
    load_tile_nt(e + start, len, acc);
  uint32_t* wb = bits + P.word_off[s] + (t - P.tile_base[s]) * (int64_t)(kTile / 32);
#pragma unroll
  for (int v = 0; v < kSlots; ++v) {
    uint32_t nib = 0;
    f4 r;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const bool neg = acc[v][c] < 0.0f;
      nib |= (neg && pb + v * 256 + c < len) ? (1u << c) : 0u;
      r[c] = acc[v][c] - (neg ? -scale : scale);
    }
    uint32_t word = nib << (4 * (lane & 7));
    word |= __shfl_xor(word, 1, 64);
    word |= __shfl_xor(word, 2, 64);
    word |= __shfl_xor(word, 4, 64);
    const int wi = (pb + v * 256) / 32;   // tile-relative word of this lane's group
    if ((lane & 7) == 0 && wi * 32 < len) wb[wi] = word;
    if (len == kTile && (start & 3) == 0) {
      f4* e4 = reinterpret_cast<f4*>(e + start);
      if (GC_NT_STORE_E) __builtin_nontemporal_store(r, e4 + ((pb + v * 256) >> 2));
      else e4[(pb + v * 256) >> 2] = r;
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (pb + v * 256 + c < len) e[start + pb + v * 256 + c] = r[c];
    }
  }
}

__global__ __launch_bounds__(kThreads) void k_sign_decompress(DevPlan P,
                                                             const uint32_t* __restrict__ bits,
                                                             const float* __restrict__ scales,
                                                             float* __restrict__ dense,
                                                             int accumulate) {
  const int64_t t = blockIdx.x;
  const int4 desc = P.tile_desc[t];
  const int64_t start = (int64_t)(((uint64_t)(uint32_t)desc.y << 32) | (uint32_t)desc.x);
  const int len = desc.z, s = desc.w;
  const float scale = scales[s];
  const int pb = slot_base(), lane = lane_id();
  const uint32_t* wb = bits + P.word_off[s] + (t - P.tile_base[s]) * (int64_t)(kTile / 32);
#pragma unroll
  for (int v = 0; v < kSlots; ++v) {
    const int wi = (pb + v * 256) / 32;
    const uint32_t nib = wi * 32 < len ? (wb[wi] >> (4 * (lane & 7))) & 0xFu : 0u;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int p = pb + v * 256 + c;
      if (p < len) {
        const float x = ((nib >> c) & 1u) ? -scale : scale;
        float* d = dense + start + p;
        *d = accumulate ? *d + x : x;
      }
    }
  }
}

// ------------------------------------------------------------------------------ QSGD
// QSGD with s levels ("Communication Optimization > Gradient Compression", QSGD paragraph,
// with the 1/s that makes E[Q] = g restored): pass 1 forms acc (e + x with error feedback,
// else x; stored only where momentum makes pass 2 unable to form it again from g and e) and
// each tile's sum of acc^2 in double; norm = fl32(sqrt(S)) per segment; pass 2
// draws the levels at step fl32(norm / s) (counter tag 0x52) and, with error feedback,
// writes e = fl(acc - fl(code * step)).

template <bool kMomentum, bool kEF>
__global__ __launch_bounds__(kThreads) void k_qsgd_pass1(DevPlan P, const float* __restrict__ g,
                                                        float* __restrict__ e,
                                                        float* __restrict__ u, float m) {
  __shared__ double s_d[kWaves];
  const int64_t t = blockIdx.x;
  const int4 desc = P.tile_desc[t];
  const int64_t start = (int64_t)(((uint64_t)(uint32_t)desc.y << 32) | (uint32_t)desc.x);
  const int len = desc.z;
  const float gf = grad_scale(P, desc.w);
  f4 acc[kSlots];
  if (kEF && kMomentum) {
    ef_add_tile<true>(g, gf, e, u, m, start, len, acc);
  } else if (kEF) {        // acc = e + g, formed again by pass 2
    acc_tile(g, gf, e, start, len, acc);
  } else if (kMomentum) {  // u = m*u + g, stored; acc = u
    const int pb = slot_base();
#pragma unroll
    for (int v = 0; v < kSlots; ++v)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int p = pb + v * 256 + c;
        float a = 0.0f;
        if (p < len) {
          const float mu = m * u[start + p];
          a = mu + g[start + p] * gf;
          u[start + p] = a;
        }
        acc[v][c] = a;
      }
  } else {
    load_tile_nt(g + start, len, acc);
#pragma unroll
    for (int v = 0; v < kSlots; ++v) acc[v] = acc[v] * gf;
  }
  double sq = 0.0;
#pragma unroll
  for (int v = 0; v < kSlots; ++v)
#pragma unroll
    for (int c = 0; c < 4; ++c) sq += (double)acc[v][c] * (double)acc[v][c];
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) sq += __shfl_xor(sq, d, 64);
  if (lane_id() == 0) s_d[wave_id()] = sq;
  __syncthreads();
  if (threadIdx.x == 0) {
    double sum = 0.0;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) sum += s_d[i];
    P.tile_l1[t] = sum;
  }
}

__global__ __launch_bounds__(1024) void k_qsgd_norm(DevPlan P, float* __restrict__ norms) {
  __shared__ double s_d[16];
  const int s = blockIdx.x;
  const int64_t t0 = P.tile_base[s], t1 = P.tile_base[s + 1];
  double sum = 0.0;
  for (int64_t t = t0 + threadIdx.x; t < t1; t += 1024) sum += P.tile_l1[t];
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) sum += __shfl_xor(sum, d, 64);
  if (lane_id() == 0) s_d[wave_id()] = sum;
  __syncthreads();
  if (threadIdx.x == 0) {
    double tot = 0.0;
    for (int i = 0; i < 16; ++i) tot += s_d[i];
    norms[s] = (float)sqrt(tot);
  }
}

// kSrc: 0 = acc in e (error feedback with momentum), 1 = acc in u (momentum, no feedback),
// 2 = acc = g, 3 = acc = e + g formed here (error feedback without momentum).
template <int kSrc>
__global__ __launch_bounds__(kThreads) void k_qsgd_pass2(DevPlan P, const float* __restrict__ g,
                                                        float* __restrict__ e,
                                                        const float* __restrict__ u,
                                                        const float* __restrict__ norms,
                                                        int levels, int8_t* __restrict__ codes,
                                                        uint32_t seed_lo, uint32_t seed_hi,
                                                        uint32_t step_lo) {
  const int64_t t = blockIdx.x;
  const int4 desc = P.tile_desc[t];
  const int64_t start = (int64_t)(((uint64_t)(uint32_t)desc.y << 32) | (uint32_t)desc.x);
  const int len = desc.z, s = desc.w;
  const float qstep = norms[s] / (float)levels;
  const float limit = (float)levels;
  const int pb = slot_base();
  f4 acc[kSlots];
  if (kSrc == 3) {
    acc_tile(g, grad_scale(P, s), e, start, len, acc);
  } else {
    load_tile_nt((kSrc == 0 ? e : (kSrc == 1 ? u : g)) + start, len, acc);
    if (kSrc == 2) {
      const float gf = grad_scale(P, s);
#pragma unroll
      for (int v = 0; v < kSlots; ++v) acc[v] = acc[v] * gf;
    }
  }
  const bool vec = len == kTile && (start & 3) == 0;
#pragma unroll
  for (int v = 0; v < kSlots; ++v) {
    f4 r;
    uint32_t packed = 0;
    // draws: word (gi % 4) of the Philox block at counter gi / 4; a lane's four elements
    // share one block when they start on a multiple of 4
    const int64_t g0 = start + pb + v * 256;
    uint32_t w[4], w2[4];
    philox4((uint32_t)(uint64_t)(g0 >> 2), (uint32_t)((uint64_t)(g0 >> 2) >> 32), step_lo, 0x52u,
            seed_lo, seed_hi, w);
    if (g0 & 3) {
      const int64_t g1 = (g0 >> 2) + 1;
      philox4((uint32_t)(uint64_t)g1, (uint32_t)((uint64_t)g1 >> 32), step_lo, 0x52u, seed_lo,
              seed_hi, w2);
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int j = (int)(g0 & 3) + c;   // position of element c from the first block
      const uint32_t word = j < 4 ? w[j] : w2[j - 4];
      float deq;
      const int code = sr_code_u24(acc[v][c], qstep, limit, word >> 8, &deq);
      packed |= ((uint32_t)(uint8_t)(int8_t)code) << (8 * c);
      r[c] = acc[v][c] - deq;
    }
    const int p0 = pb + v * 256;
    if (vec) {
      *reinterpret_cast<uint32_t*>(codes + start + p0) = packed;
      if (kSrc == 0 || kSrc == 3) {
        f4* e4 = reinterpret_cast<f4*>(e + start);
        if (GC_NT_STORE_E) __builtin_nontemporal_store(r, e4 + (p0 >> 2)); else e4[p0 >> 2] = r;
      }
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (p0 + c < len) {
          codes[start + p0 + c] = (int8_t)(packed >> (8 * c));
          if (kSrc == 0 || kSrc == 3) e[start + p0 + c] = r[c];
        }
    }
  }
}

__global__ __launch_bounds__(kThreads) void k_qsgd_decompress(DevPlan P,
                                                             const int8_t* __restrict__ codes,
                                                             const float* __restrict__ norms,
                                                             int levels,
                                                             float* __restrict__ dense,
                                                             int accumulate) {
  const int64_t t = blockIdx.x;
  const int4 desc = P.tile_desc[t];
  const int64_t start = (int64_t)(((uint64_t)(uint32_t)desc.y << 32) | (uint32_t)desc.x);
  const int len = desc.z, s = desc.w;
  const float qstep = norms[s] / (float)levels;
  const int pb = slot_base();
#pragma unroll
  for (int v = 0; v < kSlots; ++v)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int p = pb + v * 256 + c;
      if (p < len) {
        const float x = (float)codes[start + p] * qstep;
        float* d = dense + start + p;
        *d = accumulate ? *d + x : x;
      }
    }
}

// -------------------------------------------------------------------------------- Random-k
// Random-k ("Gradient Compression", memory-compression glossary, Random-k section): exactly k
// positions per segment, those with the k largest random keys (rand_key_tile), a uniformly
// random subset drawn anew each step.  The streaming pass forms acc as the Top-k pass does and
// captures by key instead of magnitude; the select and the ordered emit are shared, the kept
// values then read back from where acc lives.

// u = fl(fl(m*u) + fl(g * gf)) over one tile, stored (momentum without error feedback).
__device__ __forceinline__ void momentum_tile(const float* __restrict__ g, float gf,
                                              float* __restrict__ u, float m, int64_t start,
                                              int len) {
  const int pb = slot_base();
  if (len == kTile && (start & 3) == 0) {
    const f4* g4 = reinterpret_cast<const f4*>(g + start);
    f4* u4 = reinterpret_cast<f4*>(u + start);
    f4 gv[kSlots], uv[kSlots];
#pragma unroll
    for (int v = 0; v < kSlots; ++v) {
      const int q = (pb + v * 256) >> 2;
      gv[v] = GC_NT_LOAD_G ? __builtin_nontemporal_load(g4 + q) : g4[q];
      uv[v] = GC_NT_LOAD_E ? __builtin_nontemporal_load(u4 + q) : u4[q];
    }
#pragma unroll
    for (int v = 0; v < kSlots; ++v) {
      const int q = (pb + v * 256) >> 2;
      const f4 mu = m * uv[v];
      const f4 x = mu + gv[v] * gf;
      if (GC_NT_STORE_E) __builtin_nontemporal_store(x, u4 + q); else u4[q] = x;
    }
  } else {
#pragma unroll
    for (int v = 0; v < kSlots; ++v)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int p = pb + v * 256 + c;
        if (p < len) {
          const float mu = m * u[start + p];
          u[start + p] = mu + g[start + p] * gf;
        }
      }
  }
}

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
    }  // neither: nothing to stream, g is read at the kept positions only
    if (thr != kNoCapture) rand_key_tile(P, start, len, key);
  }
  if (thr == kNoCapture) return;  // uniform
  capture_tile(P, s, t, start, len, key, thr, s_w, &s_base);
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

// ---------------------------------------------------------------------- gradient clipping
// Local gradient clipping (genomic-FL glossary, DGC section: the gradient magnitude is
// normalised before compression), per segment: norm = fl32(sqrt(sum g^2)) (k_qsgd_pass1 and
// k_qsgd_norm on g), then where norm > c: g = fl(g * fl32(c / norm)).  Tiles of segments
// that are not clipped are left untouched (no write).
__global__ __launch_bounds__(kThreads) void k_clip_scale(DevPlan P, float* __restrict__ g,
                                                        const float* __restrict__ max_norm,
                                                        const float* __restrict__ norms) {
  const int64_t t = blockIdx.x;
  const int4 desc = P.tile_desc[t];
  const int64_t start = (int64_t)(((uint64_t)(uint32_t)desc.y << 32) | (uint32_t)desc.x);
  const int len = desc.z, s = desc.w;
  const float norm = norms[s], c = max_norm[s];
  if (!(norm > c)) return;   // uniform per tile
  const float f = c / norm;
  const int pb = slot_base();
  if (len == kTile && (start & 3) == 0) {
    f4* g4 = reinterpret_cast<f4*>(g + start);
    f4 x[kSlots];
#pragma unroll
    for (int v = 0; v < kSlots; ++v) x[v] = __builtin_nontemporal_load(g4 + ((pb + v * 256) >> 2));
#pragma unroll
    for (int v = 0; v < kSlots; ++v)
      __builtin_nontemporal_store(x[v] * f, g4 + ((pb + v * 256) >> 2));
  } else {
#pragma unroll
    for (int v = 0; v < kSlots; ++v)
#pragma unroll
      for (int c4 = 0; c4 < 4; ++c4) {
        const int p = pb + v * 256 + c4;
        if (p < len) g[start + p] = g[start + p] * f;
      }
  }
}

// Per segment: the clipping factor fl32(c / norm) where norm > c, else 1 (the scale that a
// later compress call applies to g on load, when the plan carries it).
__global__ __launch_bounds__(kThreads) void k_clip_factor(int32_t n_seg,
                                                         const float* __restrict__ max_norm,
                                                         const float* __restrict__ norms,
                                                         float* __restrict__ factors) {
  const int s = blockIdx.x * kThreads + threadIdx.x;
  if (s >= n_seg) return;
  const float norm = norms[s], c = max_norm[s];
  factors[s] = norm > c ? c / norm : 1.0f;
}

// ------------------------------------------------------------------------------ int8 stage
// Per segment: scale = fl(max |v| / 127) over the kept values.
__global__ __launch_bounds__(1024) void k_absmax(OutPlan O, const float* __restrict__ vals,
                                                 float* __restrict__ scales) {
  __shared__ uint32_t s_m[16];
  const int s = blockIdx.x;
  const int64_t a = O.out_off[s], b = O.out_off[s + 1];
  uint32_t mx = 0;
  for (int64_t j = a + threadIdx.x; j < b; j += 1024) mx = max(mx, mag_key(vals[j]));
  for (int d = 32; d >= 1; d >>= 1) mx = max(mx, (uint32_t)__shfl_xor(mx, d, 64));
  if (lane_id() == 0) s_m[wave_id()] = mx;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t m = 0;
    for (int i = 0; i < 16; ++i) m = max(m, s_m[i]);
    scales[s] = __uint_as_float(m) / 127.0f;
  }
}

__global__ __launch_bounds__(kThreads) void k_quant(OutPlan O, const float* __restrict__ vals,
                                                    const int32_t* __restrict__ idx,
                                                    float* __restrict__ e, uint32_t seed_lo,
                                                    uint32_t seed_hi, uint32_t step_lo,
                                                    int8_t* __restrict__ codes,
                                                    const float* __restrict__ scales) {
  const int64_t ch = blockIdx.x;
  const int s = O.out_chunk_seg[ch];
  const int64_t j0 = O.out_off[s] + (ch - O.out_chunk_base[s]) * (int64_t)kOutChunk;
  const int64_t j1 = min(j0 + kOutChunk, O.out_off[s + 1]);
  const float scale = scales[s];
  const int64_t s0 = O.seg_off[s], n_s = O.seg_off[s + 1] - s0;
  for (int64_t j = j0 + threadIdx.x; j < j1; j += kThreads) {
    const float v = vals[j];
    const int32_t li = idx[j];
    const int64_t gi = s0 + li;
    float deq;
    const int code = quant_code(v, scale, gi, seed_lo, seed_hi, step_lo, &deq);
    codes[j] = (int8_t)code;
    if (e && li >= 0 && li < n_s) e[gi] = v - deq;  // indices come from the compress call
  }
}

// ---------------------------------------------------------------------------- decompress
__global__ __launch_bounds__(kThreads) void k_fill_zero(float* __restrict__ d, int64_t a,
                                                        int64_t b) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t i = a + (int64_t)blockIdx.x * kThreads + threadIdx.x; i < b; i += stride)
    d[i] = 0.0f;
}

__global__ __launch_bounds__(kThreads) void k_scatter_out(OutPlan O,
                                                          const float* __restrict__ vals,
                                                          const int8_t* __restrict__ codes,
                                                          const float* __restrict__ scales,
                                                          const int32_t* __restrict__ idx,
                                                          float* __restrict__ dense,
                                                          int accumulate) {
  const int64_t ch = blockIdx.x;
  const int s = O.out_chunk_seg[ch];
  const int64_t j0 = O.out_off[s] + (ch - O.out_chunk_base[s]) * (int64_t)kOutChunk;
  const int64_t j1 = min(j0 + kOutChunk, O.out_off[s + 1]);
  const int64_t s0 = O.seg_off[s], n_s = O.seg_off[s + 1] - s0;
  const float scale = vals ? 0.0f : scales[s];
  for (int64_t j = j0 + threadIdx.x; j < j1; j += kThreads) {
    const float v = vals ? vals[j] : (float)codes[j] * scale;
    const int32_t li = idx[j];
    if (li < 0 || li >= n_s) continue;  // indices come from the compress call
    float* d = dense + s0 + li;
    *d = accumulate ? *d + v : v;
  }
}

// --------------------------------------------------------------------------------- copy
__global__ __launch_bounds__(kThreads) void k_copy(const f4* __restrict__ src,
                                                   f4* __restrict__ dst, int64_t n4) {
  const int64_t block = (int64_t)blockIdx.x * (kThreads * kSlots);
  const int64_t base = block + threadIdx.x;
  f4 x[kSlots];
  if (block + kThreads * kSlots <= n4) {
#pragma unroll
    for (int v = 0; v < kSlots; ++v) x[v] = __builtin_nontemporal_load(src + base + v * kThreads);
#pragma unroll
    for (int v = 0; v < kSlots; ++v) dst[base + v * kThreads] = x[v];
    return;
  }
  for (int v = 0; v < kSlots; ++v) {
    const int64_t i = base + v * kThreads;
    if (i < n4) dst[i] = src[i];
  }
}

inline unsigned blocks_for(int64_t n, int per) { return (unsigned)((n + per - 1) / per); }

// Everything after the streaming pass: select (candidates, re-capture or the exact full
// path), ordered count/scan, emit.  e holds acc (magnitude keys); scales: fused int8 or null.
void select_emit(const DevPlan& P, const float* e, const EmitOut& o, float* scales,
                 hipStream_t st) {
  k_select_init<<<P.n_seg, kThreads, 0, st>>>(P);
  k_recap_hist<<<kFullBlocks, kThreads, 0, st>>>(P, e);
  k_recap_decide<<<P.n_seg, kThreads, 0, st>>>(P);
  k_recapture<<<kFullBlocks, kThreads, 0, st>>>(P, e);
  k_runs<<<P.n_seg, 1024, 0, st>>>(P);
  if (P.n_chunks > 0) k_scatter<<<(unsigned)P.n_chunks, kThreads, 0, st>>>(P);
  k_find<<<P.n_seg, kThreads, 0, st>>>(P, 0);
  const unsigned mixed = (unsigned)(P.n_chunks + kFullBlocks);
  for (int pass = 1; pass < 3; ++pass) {
    k_hist<<<mixed, kThreads, 0, st>>>(P, e, pass);
    k_find<<<P.n_seg, kThreads, 0, st>>>(P, pass);
  }
  if (P.n_chunks > 0) k_count_cand<<<(unsigned)P.n_chunks, kThreads, 0, st>>>(P);
  k_count_full<<<kFullBlocks, kThreads, 0, st>>>(P, e);
  k_scan<<<P.n_seg, 1024, 0, st>>>(P, scales);
  if (P.n_chunks > 0) k_emit_cand<<<(unsigned)P.n_chunks, kThreads, 0, st>>>(P, o);
  k_emit_full<<<kFullBlocks, kThreads, 0, st>>>(P, o);
}

}  // namespace

hipError_t launch_compress(const DevPlan& P, const float* g, float* e, float* u, float m,
                           float* out_vals, int32_t* out_idx, const Int8Args& q8,
                           hipStream_t st, hipEvent_t ev_begin, hipEvent_t ev_end) {
  if (P.n_seg == 0) return hipSuccess;
  k_prep<<<blocks_for(P.n_seg, kThreads), kThreads, 0, st>>>(P);
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
      else k_randk_capture<false, false><<<nt, kThreads, 0, st>>>(Q, g, nullptr, nullptr, m);
    } else {
      if (e && u) k_randk_capture<true, true><<<nt, kThreads, 0, st>>>(Q, g, e, u, m);
      else if (e) k_randk_capture<false, true><<<nt, kThreads, 0, st>>>(Q, g, e, nullptr, m);
      else if (u) k_randk_capture<true, false><<<nt, kThreads, 0, st>>>(Q, g, nullptr, u, m);
      else k_randk_capture<false, false><<<nt, kThreads, 0, st>>>(Q, g, nullptr, nullptr, m);
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


hipError_t launch_sign(const DevPlan& P, const float* g, float* e, float* u, float m,
                       uint32_t* bits, float* scales, hipStream_t st, hipEvent_t ev_begin,
                       hipEvent_t ev_end) {
  if (P.n_seg == 0) return hipSuccess;
  if (ev_begin) (void)hipEventRecord(ev_begin, st);
  if (P.n_tiles > 0) {
    if (u)
      k_sign_pass1<true><<<(unsigned)P.n_tiles, kThreads, 0, st>>>(P, g, e, u, m);
    else
      k_sign_pass1<false><<<(unsigned)P.n_tiles, kThreads, 0, st>>>(P, g, e, nullptr, m);
  }
  k_sign_scale<<<P.n_seg, 1024, 0, st>>>(P, scales);
  if (P.n_tiles > 0) {
    if (u)
      k_sign_pass2<false><<<(unsigned)P.n_tiles, kThreads, 0, st>>>(P, g, e, bits, scales);
    else
      k_sign_pass2<true><<<(unsigned)P.n_tiles, kThreads, 0, st>>>(P, g, e, bits, scales);
  }
  if (ev_end) (void)hipEventRecord(ev_end, st);
  return hipGetLastError();
}

hipError_t launch_sign_decompress(const DevPlan& P, const uint32_t* bits, const float* scales,
                                  float* dense, int accumulate, hipStream_t st) {
  if (P.n_tiles == 0) return hipSuccess;
  k_sign_decompress<<<(unsigned)P.n_tiles, kThreads, 0, st>>>(P, bits, scales, dense,
                                                             accumulate);
  return hipGetLastError();
}

hipError_t launch_qsgd(const DevPlan& P, const float* g, float* e, float* u, float m,
                       int levels, uint64_t seed, uint64_t step, int8_t* codes, float* norms,
                       hipStream_t st, hipEvent_t ev_begin, hipEvent_t ev_end) {
  if (P.n_seg == 0) return hipSuccess;
  const unsigned nt = (unsigned)P.n_tiles;
  if (ev_begin) (void)hipEventRecord(ev_begin, st);
  if (nt > 0) {
    if (e && u) k_qsgd_pass1<true, true><<<nt, kThreads, 0, st>>>(P, g, e, u, m);
    else if (e) k_qsgd_pass1<false, true><<<nt, kThreads, 0, st>>>(P, g, e, nullptr, m);
    else if (u) k_qsgd_pass1<true, false><<<nt, kThreads, 0, st>>>(P, g, nullptr, u, m);
    else k_qsgd_pass1<false, false><<<nt, kThreads, 0, st>>>(P, g, nullptr, nullptr, m);
  }
  k_qsgd_norm<<<P.n_seg, 1024, 0, st>>>(P, norms);
  if (nt > 0) {
    const uint32_t sl = (uint32_t)seed, sh = (uint32_t)(seed >> 32), tl = (uint32_t)step;
    if (e && u) k_qsgd_pass2<0><<<nt, kThreads, 0, st>>>(P, g, e, u, norms, levels, codes, sl, sh, tl);
    else if (e) k_qsgd_pass2<3><<<nt, kThreads, 0, st>>>(P, g, e, u, norms, levels, codes, sl, sh, tl);
    else if (u) k_qsgd_pass2<1><<<nt, kThreads, 0, st>>>(P, g, e, u, norms, levels, codes, sl, sh, tl);
    else k_qsgd_pass2<2><<<nt, kThreads, 0, st>>>(P, g, e, u, norms, levels, codes, sl, sh, tl);
  }
  if (ev_end) (void)hipEventRecord(ev_end, st);
  return hipGetLastError();
}

hipError_t launch_qsgd_decompress(const DevPlan& P, const int8_t* codes, const float* norms,
                                  int levels, float* dense, int accumulate, hipStream_t st) {
  if (P.n_tiles == 0) return hipSuccess;
  k_qsgd_decompress<<<(unsigned)P.n_tiles, kThreads, 0, st>>>(P, codes, norms, levels, dense,
                                                             accumulate);
  return hipGetLastError();
}

hipError_t launch_clip(const DevPlan& P, float* g, const float* max_norm, float* norms,
                       float* factors, hipStream_t st) {
  if (P.n_seg == 0) return hipSuccess;
  DevPlan Q = P;
  Q.gscale = nullptr;   // the norm is the raw gradient's
  const unsigned nt = (unsigned)Q.n_tiles;
  if (nt > 0) k_qsgd_pass1<false, false><<<nt, kThreads, 0, st>>>(Q, g, nullptr, nullptr, 0.0f);
  k_qsgd_norm<<<Q.n_seg, 1024, 0, st>>>(Q, norms);
  if (factors)
    k_clip_factor<<<blocks_for(Q.n_seg, kThreads), kThreads, 0, st>>>(Q.n_seg, max_norm, norms,
                                                                      factors);
  else if (nt > 0)
    k_clip_scale<<<nt, kThreads, 0, st>>>(Q, g, max_norm, norms);
  return hipGetLastError();
}

hipError_t launch_reset(const DevPlan& P, hipStream_t st) {
  if (P.n_seg == 0) return hipSuccess;
  k_reset<<<blocks_for(P.n_seg, kThreads), kThreads, 0, st>>>(P);
  return hipGetLastError();
}

hipError_t launch_quant(const OutPlan& O, const float* vals, const int32_t* idx, float* e,
                        uint64_t seed, uint64_t step, int8_t* codes, float* scales,
                        hipStream_t st) {
  if (O.n_seg == 0) return hipSuccess;
  k_absmax<<<O.n_seg, 1024, 0, st>>>(O, vals, scales);
  if (O.n_out_chunks > 0)
    k_quant<<<(unsigned)O.n_out_chunks, kThreads, 0, st>>>(
        O, vals, idx, e, (uint32_t)seed, (uint32_t)(seed >> 32), (uint32_t)step, codes, scales);
  return hipGetLastError();
}

hipError_t launch_decompress(const OutPlan& O, const float* vals, const int8_t* codes,
                             const float* scales, const int32_t* idx, float* dense,
                             int accumulate, hipStream_t st) {
  if (O.n_seg == 0) return hipSuccess;
  if (O.n_out_chunks > 0)
    k_scatter_out<<<(unsigned)O.n_out_chunks, kThreads, 0, st>>>(O, vals, codes, scales, idx,
                                                                 dense, accumulate);
  return hipGetLastError();
}

hipError_t launch_fill_zero(float* dense, int64_t a, int64_t b, hipStream_t st) {
  if (b <= a) return hipSuccess;
  const int64_t want = (b - a + kThreads - 1) / kThreads;
  const unsigned blocks = (unsigned)(want < 65536 ? want : 65536);
  k_fill_zero<<<blocks, kThreads, 0, st>>>(dense, a, b);
  return hipGetLastError();
}

hipError_t launch_copy(const float* src, float* dst, int64_t n, hipStream_t st) {
  const int64_t n4 = n / 4;
  if (n4 == 0) return hipSuccess;
  k_copy<<<blocks_for(n4, kThreads * kSlots), kThreads, 0, st>>>(
      reinterpret_cast<const f4*>(src), reinterpret_cast<f4*>(dst), n4);
  return hipGetLastError();
}

}  // namespace gc
