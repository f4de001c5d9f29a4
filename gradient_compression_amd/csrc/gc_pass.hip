// gc_pass.hip -- the streaming pass of the error-feedback Top-k and threshold calls, on its
// own: one read of g and e (and u), one write of acc into e (and u), and the capture of the
// candidates.  Kept apart from the kernels after it so that a change to those leaves the
// pass's code, and the HBM counters taken on it, as they are.
//
// The method is the Top-K with error feedback of "Communication Optimization > Gradient
// Compression" (Top-K section equations); momentum correction per the "Gradient
// Sparsification" glossary.
#include "gc_capture.h"

#pragma clang fp contract(off)

namespace gc {
namespace {

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
  reset_call_lists(P);

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
    const uint32_t tk = mag_key(P.tau[s]);
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
  const uint32_t thr = kCountTau ? capture_thr(P, s) : P.thr[s];
  if (thr == kNoCapture) return;  // uniform: nothing to capture (small, or not estimated yet)
  capture_tile(P, s, t, start, len, acc, thr, &P.cand_cnt[s], s_w, &s_base);
}

}  // namespace

void launch_ef_capture(const DevPlan& P, const float* g, float* e, float* u, float m,
                       bool count_tau, hipStream_t st) {
  if (P.n_tiles <= 0) return;
  const unsigned nt = (unsigned)P.n_tiles;
  if (count_tau) {
    if (P.gscale) {
      if (u) k_ef_capture<true, true, true><<<nt, kThreads, 0, st>>>(P, g, e, u, m);
      else k_ef_capture<false, true, true><<<nt, kThreads, 0, st>>>(P, g, e, nullptr, m);
    } else {
      if (u) k_ef_capture<true, true><<<nt, kThreads, 0, st>>>(P, g, e, u, m);
      else k_ef_capture<false, true><<<nt, kThreads, 0, st>>>(P, g, e, nullptr, m);
    }
  } else {
    if (P.gscale) {
      if (u) k_ef_capture<true, false, true><<<nt, kThreads, 0, st>>>(P, g, e, u, m);
      else k_ef_capture<false, false, true><<<nt, kThreads, 0, st>>>(P, g, e, nullptr, m);
    } else {
      if (u) k_ef_capture<true><<<nt, kThreads, 0, st>>>(P, g, e, u, m);
      else k_ef_capture<false><<<nt, kThreads, 0, st>>>(P, g, e, nullptr, m);
    }
  }
}

}  // namespace gc
