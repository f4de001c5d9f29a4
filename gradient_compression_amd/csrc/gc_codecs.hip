// gc_codecs.hip -- gfx950 kernels of the two-pass codecs (1-bit sign with error feedback,
// QSGD with s levels) and of local gradient clipping: a streaming pass for the per-segment
// sum (|acc| or acc^2, in double), the per-segment scale, then a streaming pass that writes the
// codes and the residual (or scales g).
#include "gc_random.h"

#pragma clang fp contract(off)

namespace gc {
namespace {

// ------------------------------------------------------------------------ 1-bit sign
// 1-bit sign compression with error feedback ("Communication Optimization > Gradient
// Compression", 1-bit SGD section: Q(g) = sign(g) * ||g||_1 / d, one scale per layer; error
// feedback as for top-K).  Pass 1 takes each tile's sum of |acc| in double (with momentum it
// also stores u and acc = e + u; without, it only reads and pass 2 forms acc = e + g again);
// the scale is fl32(S / n) per segment; pass 2 writes the sign bits (bit i of word i/32,
// 1 = negative) and the residual e = fl(acc - sign * scale).

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

}  // namespace

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

}  // namespace gc
