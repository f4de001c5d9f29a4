// gc_scatter.hip -- gfx950 kernels over the compressed payloads: the int8 stage of kept
// values (per-segment absmax, Philox stochastic rounding, quantisation error fed back),
// decompression into a dense buffer, and the reference copy and y += x streams used to
// calibrate bandwidth.
#include "gc_random.h"

#pragma clang fp contract(off)

namespace gc {
namespace {

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

// ------------------------------------------------------------------------------ add
// y = fl(y + x) with the streaming pass's memory pattern and none of its other work: the same
// tile layout, non-temporal dwordx4 loads of both inputs and a non-temporal store of y.  A
// reference 2-read/1-write stream (the pass itself streams faster than this bare kernel, so it
// is not a ceiling).
__global__ __launch_bounds__(kThreads) void k_add(const float* __restrict__ x,
                                                  float* __restrict__ y, int64_t n) {
  const int64_t start = (int64_t)blockIdx.x * kTile;
  const int64_t rem = n - start;
  const int len = rem < kTile ? (int)rem : kTile;
  const int pb = slot_base();
  if (len == kTile) {
    const f4* x4 = reinterpret_cast<const f4*>(x + start);
    f4* y4 = reinterpret_cast<f4*>(y + start);
    f4 a[kSlots], b[kSlots];
#pragma unroll
    for (int v = 0; v < kSlots; ++v) {
      a[v] = __builtin_nontemporal_load(x4 + ((pb + v * 256) >> 2));
      b[v] = __builtin_nontemporal_load(y4 + ((pb + v * 256) >> 2));
    }
#pragma unroll
    for (int v = 0; v < kSlots; ++v) __builtin_nontemporal_store(b[v] + a[v], y4 + ((pb + v * 256) >> 2));
    return;
  }
#pragma unroll
  for (int v = 0; v < kSlots; ++v)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int p = pb + v * 256 + c;
      if (p < len) y[start + p] = y[start + p] + x[start + p];
    }
}

// ----------------------------------------------------------------------------- read
// A pure read stream in the pass's tile layout: non-temporal dwordx4 loads of x, folded into
// an xor of the bit patterns, which is stored only if it equals a value no real stream of
// floats produces here (so the loads cannot be dropped and nothing is written).
__global__ __launch_bounds__(kThreads) void k_read(const float* __restrict__ x, int64_t n,
                                                   uint32_t* __restrict__ sink) {
  const int64_t start = (int64_t)blockIdx.x * kTile;
  const int64_t rem = n - start;
  const int len = rem < kTile ? (int)rem : kTile;
  const int pb = slot_base();
  uint32_t h = 0;
  if (len == kTile) {
    const f4* x4 = reinterpret_cast<const f4*>(x + start);
    f4 a[kSlots];
#pragma unroll
    for (int v = 0; v < kSlots; ++v) a[v] = __builtin_nontemporal_load(x4 + ((pb + v * 256) >> 2));
#pragma unroll
    for (int v = 0; v < kSlots; ++v)
#pragma unroll
      for (int c = 0; c < 4; ++c) h ^= __float_as_uint(a[v][c]);
  } else {
#pragma unroll
    for (int v = 0; v < kSlots; ++v)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int p = pb + v * 256 + c;
        if (p < len) h ^= __float_as_uint(x[start + p]);
      }
  }
  if (h == 0x7FC0A5A5u) sink[threadIdx.x & 63] = h;
}

}  // namespace

hipError_t launch_read(const float* x, int64_t n, uint32_t* sink, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  k_read<<<blocks_for(n, kTile), kThreads, 0, st>>>(x, n, sink);
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

hipError_t launch_add(const float* x, float* y, int64_t n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  k_add<<<blocks_for(n, kTile), kThreads, 0, st>>>(x, y, n);
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
