// gc_device.h -- device-side building blocks shared by the gfx950 kernels: the tile layout
// and its ordered ranks (ballots, mbcnt, LDS prefixes), block scans, Philox4x32-10, stochastic
// rounding, the streaming loads of a tile (with the error-feedback add, momentum and the
// optional gradient scale) and the Random-k keys.  Included by each kernel source.
#pragma once

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

// Exclusive scans of two uint32 per thread at once (one pair of barriers); *ta and *tb get the
// sums.  s_a, s_b: __shared__ uint32_t[NT / 64] each.  Contains barriers.
template <int NT>
__device__ void block_excl_scan2(uint32_t a, uint32_t b, uint32_t* s_a, uint32_t* s_b,
                                 uint32_t* ea, uint32_t* eb, uint32_t* ta, uint32_t* tb) {
  const int lane = lane_id(), w = wave_id();
  uint32_t x = a, y = b;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t px = __shfl_up(x, d, 64), py = __shfl_up(y, d, 64);
    if (lane >= d) {
      x += px;
      y += py;
    }
  }
  if (lane == 63) {
    s_a[w] = x;
    s_b[w] = y;
  }
  __syncthreads();
  uint32_t ba = 0, bb = 0, sa = 0, sb = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) {
    const uint32_t u = s_a[i], v = s_b[i];
    ba += (i < w) ? u : 0u;
    bb += (i < w) ? v : 0u;
    sa += u;
    sb += v;
  }
  __syncthreads();
  *ea = ba + x - a;
  *eb = bb + y - b;
  *ta = sa;
  *tb = sb;
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
__device__ inline uint32_t tile_rank(const uint32_t (&bits)[kSlots], uint32_t (&woff)[kSlots],
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

inline unsigned blocks_for(int64_t n, int per) { return (unsigned)((n + per - 1) / per); }

}  // namespace
}  // namespace gc
