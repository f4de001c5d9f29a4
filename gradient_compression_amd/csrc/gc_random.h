// gc_random.h -- the counter-based random numbers of the codecs (Philox4x32-10, Salmon et al.,
// SC'11, from its published definition), the stochastic rounding built on them, and the
// Random-k keys.  Not included by the streaming pass of the Top-k path, which draws nothing.
#pragma once
#include "gc_device.h"

namespace gc {
namespace {

// Three-input XOR in one instruction (gfx950's three-input bitwise op, truth table 0x96).
__device__ __forceinline__ uint32_t xor3(uint32_t a, uint32_t b, uint32_t c) {
  return __builtin_amdgcn_bitop3_b32(a, b, c, 0x96);
}

// Philox4x32-10 (Salmon et al., SC'11), word 0 of the output block.
__device__ __forceinline__ uint32_t philox_word0(uint32_t c0, uint32_t c1, uint32_t c2,
                                                 uint32_t c3, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int round = 0; round < 10; ++round) {
    // one 32x32->64 product per multiplier (a single v_mad_u64_u32 gives both halves)
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0, p1 = (uint64_t)0xCD9E8D57u * c2;
    const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    const uint32_t n0 = xor3(hi1, c1, k0), n2 = xor3(hi0, c3, k1);
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
    const uint32_t n0 = xor3(hi1, c1, k0), n2 = xor3(hi0, c3, k1);
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

// The Random-k keys of the four elements from global index g0: word (gi % 4) of the
// Philox4x32-10 block keyed (seed lo, seed hi) at counter (gi / 4 lo, gi / 4 hi, step lo, 0x53),
// shifted right by one (31 bits).  The four share one block when g0 is a multiple of 4
// (kAligned: the caller knows that it is).
template <bool kAligned = false>
__device__ __forceinline__ void rand_key4(const DevPlan& P, int64_t g0, uint32_t (&k)[4]) {
  const uint64_t b0 = (uint64_t)g0 >> 2;
  uint32_t w[4], w2[4];
  philox4((uint32_t)b0, (uint32_t)(b0 >> 32), P.step_lo, 0x53u, P.seed_lo, P.seed_hi, w);
  if (kAligned || (g0 & 3) == 0) {   // the four elements are the block's four words
#pragma unroll
    for (int c = 0; c < 4; ++c) k[c] = w[c] >> 1;
    return;
  }
  philox4((uint32_t)(b0 + 1), (uint32_t)((b0 + 1) >> 32), P.step_lo, 0x53u, P.seed_lo,
          P.seed_hi, w2);
  // element c is word (g0 % 4) + c of the two blocks, selected with constant indices only so
  // that w and w2 stay in registers
  const int a = (int)(g0 & 3);
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int j = a + c;
    const uint32_t word = j == 0 ? w[0] : j == 1 ? w[1] : j == 2 ? w[2] : j == 3 ? w[3]
                        : j == 4 ? w2[0] : j == 5 ? w2[1] : w2[2];
    k[c] = word >> 1;
  }
}

// Random-k keys of the len (<= kTile) elements from global index start, in the tile layout,
// as float bit patterns (rand_key4 per slot).  Lanes past len get key 0.
__device__ __forceinline__ void rand_key_tile(const DevPlan& P, int64_t start, int len,
                                              f4 (&x)[kSlots]) {
  const int pb = slot_base();
#pragma unroll
  for (int v = 0; v < kSlots; ++v) {
    uint32_t k[4];
    rand_key4(P, start + pb + v * 256, k);
#pragma unroll
    for (int c = 0; c < 4; ++c) x[v][c] = pb + v * 256 + c < len ? __uint_as_float(k[c]) : 0.0f;
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

}  // namespace
}  // namespace gc
