// gc_api.hip -- host side of the C ABI declared in include/gc.h: plan construction (segment,
// tile and chunk tables, candidate capacities, device workspace), argument checks, and the
// launch sequence of each entry point.  No call except gc_plan_create allocates device memory.
#include "gc.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <initializer_list>
#include <memory>
#include <mutex>
#include <new>
#include <utility>
#include <vector>

#include "gc_internal.h"

namespace gc {
// The reference streams of gc_add_f32 and gc_read_f32 (gc_scatter.hip).
hipError_t launch_add(const float* x, float* y, int64_t n, hipStream_t st);
hipError_t launch_read(const float* x, int64_t n, uint32_t* sink, hipStream_t st);
}  // namespace gc

namespace {

// Candidate capacity of a larger segment, in multiples of its k (at least kMinCapacity).
constexpr int64_t kCapacityFactor = 16;
constexpr int64_t kMinCapacity = 65536;
// Tiles per segment that the cold-start sample reads (about 0.5M elements).
constexpr int64_t kSampleTiles = 64;

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Random-k capture threshold of a segment whose candidates do not cover it whole: the count
// of 31-bit uniform keys at or above it has mean at least mu = k + 12 sqrt(k) + 64, so by the
// Chernoff bound fewer than k of them (the exact fallback then runs) has probability below
// exp(-(mu - k)^2 / (2 mu)) < e^-37 for every k >= 1, and more than the capacity of
// max(16 k, 65536) is rarer still.
uint32_t randk_threshold(int64_t n, int64_t k) {
  const double want = (double)k + 12.0 * std::sqrt((double)k) + 64.0;
  if (want >= (double)n) return 0;
  const double span = std::ceil(want * 2147483648.0 / (double)n);
  return span >= 2147483648.0 ? 0u : (uint32_t)(2147483648.0 - span);
}
inline int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// k = min(n, ceil(n * ratio)) with the ratio in exact parts per billion; -1 if invalid.
int64_t k_from_ratio(int64_t n, double ratio) {
  if (!(ratio >= 0.0 && ratio <= 1.0)) return -1;
  if (n <= 0) return 0;
  const int64_t ppb = std::llround(ratio * 1e9);
  const __int128 num = (__int128)n * ppb + 999999999;
  const int64_t k = (int64_t)(num / 1000000000);
  return std::min(k, n);
}

struct Carver {  // sub-allocates one device block, 256-byte aligned pieces
  size_t off = 0;
  std::vector<std::pair<void**, size_t>> req;
  template <typename T>
  void add(T** p, int64_t count) {
    req.emplace_back(reinterpret_cast<void**>(p), (size_t)std::max<int64_t>(count, 1) * sizeof(T));
  }
  size_t total() const {
    size_t t = 0;
    for (auto& r : req) t += (r.second + 255) & ~(size_t)255;
    return t;
  }
  void place(char* base) {
    size_t o = 0;
    for (auto& r : req) {
      *r.first = base + o;
      o += (r.second + 255) & ~(size_t)255;
    }
  }
};

}  // namespace

struct gc_plan {
  int device = 0;
  int32_t n_seg = 0;
  uint32_t flags = 0;
  std::vector<int64_t> seg_off, k, out_off, word_off;
  int64_t total_k = 0;
  gc::DevPlan dp{};
  gc::OutPlan op{};
  void* mem = nullptr;
  bool timing = false;
  bool cold = true;   // no threshold estimate yet (fresh plan, or after a reset)
  std::vector<std::pair<hipEvent_t, hipEvent_t>> pending, spare;
};

namespace {

int check_device(const gc_plan* p) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return GC_ERR_HIP;
  return dev == p->device ? GC_OK : GC_ERR_INVALID_ARG;
}

template <typename T>
hipError_t upload(T* dst, const std::vector<T>& src) {
  if (src.empty()) return hipSuccess;
  return hipMemcpy(dst, src.data(), src.size() * sizeof(T), hipMemcpyHostToDevice);
}

// The bytes a call touches through one pointer.  Dense buffers are indexed by the absolute
// offsets of the segment table, so they span [seg_off[0], seg_off[n_seg]) elements.
struct Span {
  const void* p;
  uint64_t bytes;
};
Span dense_span(const gc_plan* plan, const void* p, uint64_t elt) {
  if (!p) return {nullptr, 0};
  const int64_t lo = plan->seg_off[0], hi = plan->seg_off[plan->n_seg];
  return {static_cast<const char*>(p) + lo * (int64_t)elt, (uint64_t)(hi - lo) * elt};
}
Span flat(const void* p, int64_t count, uint64_t elt) {
  return {p, p ? (uint64_t)count * elt : 0};
}
// True when two of the spans share a byte (NULL and empty spans share none).
bool any_overlap(std::initializer_list<Span> spans) {
  for (const Span* a = spans.begin(); a != spans.end(); ++a)
    for (const Span* b = a + 1; b != spans.end(); ++b) {
      if (!a->bytes || !b->bytes) continue;
      const uintptr_t a0 = reinterpret_cast<uintptr_t>(a->p);
      const uintptr_t b0 = reinterpret_cast<uintptr_t>(b->p);
      if (a0 < b0 + b->bytes && b0 < a0 + a->bytes) return true;
    }
  return false;
}

}  // namespace

extern "C" {

const char* gc_status_string(int status) {
  switch (status) {
    case GC_OK: return "success";
    case GC_ERR_INVALID_ARG: return "invalid argument";
    case GC_ERR_OOM: return "out of device memory";
    case GC_ERR_HIP: return "HIP runtime error";
    case GC_ERR_UNSUPPORTED: return "unsupported request";
    default: return "unknown status";
  }
}

int gc_layout(const int64_t* seg_off, int32_t n_seg, const int64_t* k, const double* ratio,
              int64_t* k_out, int64_t* out_off) {
  if (n_seg < 0 || !seg_off) return GC_ERR_INVALID_ARG;
  if (n_seg > 0 && (k == nullptr) == (ratio == nullptr)) return GC_ERR_INVALID_ARG;
  if (seg_off[0] < 0) return GC_ERR_INVALID_ARG;
  int64_t total = 0;
  for (int32_t s = 0; s < n_seg; ++s) {
    const int64_t n = seg_off[s + 1] - seg_off[s];
    if (n < 0 || n > INT32_MAX) return GC_ERR_INVALID_ARG;
    const int64_t ks = k ? k[s] : k_from_ratio(n, ratio[s]);
    if (ks < 0 || ks > n) return GC_ERR_INVALID_ARG;
    if (k_out) k_out[s] = ks;
    if (out_off) out_off[s] = total;
    total += ks;
  }
  if (out_off) out_off[n_seg] = total;
  return GC_OK;
}

}  // extern "C"

namespace {

// gc_plan_create's work; host allocations may throw std::bad_alloc, which the entry point
// turns into GC_ERR_OOM.  The device workspace is allocated after the last host allocation,
// so a throw never leaves it behind.
int plan_create(const int64_t* seg_off, int32_t n_seg, const int64_t* k, const double* ratio,
                uint32_t flags, gc_plan** out) {
  std::vector<int64_t> ks(n_seg);
  if (int rc = gc_layout(seg_off, n_seg, k, ratio, ks.data(), nullptr)) return rc;

  std::unique_ptr<gc_plan> p(new gc_plan());
  if (hipGetDevice(&p->device) != hipSuccess) return GC_ERR_HIP;
  p->n_seg = n_seg;
  p->flags = flags;
  p->seg_off.assign(seg_off, seg_off + n_seg + 1);
  p->k = ks;
  p->out_off.assign(n_seg + 1, 0);
  for (int32_t s = 0; s < n_seg; ++s) p->out_off[s + 1] = p->out_off[s] + ks[s];
  p->total_k = p->out_off[n_seg];
  p->word_off.assign(n_seg + 1, 0);
  for (int32_t s = 0; s < n_seg; ++s)
    p->word_off[s + 1] = p->word_off[s] + ceil_div(seg_off[s + 1] - seg_off[s], 32);

  // tables
  std::vector<int64_t> tile_base(n_seg + 1, 0), chunk_base(n_seg + 1, 0), cand_base(n_seg, 0),
      out_chunk_base(n_seg + 1, 0);
  std::vector<uint32_t> kk(n_seg), cap(n_seg), thr_init(n_seg), thr_rand(n_seg),
      seg_flags(n_seg, 0);
  std::vector<float> rk_scale(n_seg, 0.0f);
  int64_t cand_total = 0;
  const bool no_estimate = (flags & (GC_DEBUG_FORCE_FALLBACK | GC_DEBUG_NO_ESTIMATE)) != 0;
  for (int32_t s = 0; s < n_seg; ++s) {
    const int64_t n = seg_off[s + 1] - seg_off[s];
    tile_base[s + 1] = tile_base[s] + ceil_div(n, gc::kTile);
    int64_t c = 0;
    uint32_t thr = gc::kNoCapture, thr_r = gc::kNoCapture;
    if (n <= gc::kSmallSegment) {
      // selected whole by one workgroup of the select kernel: no capture, no candidates
      seg_flags[s] = gc::kSegSmall;
    } else if (ks[s] > 0) {
      if (ks[s] * kCapacityFactor >= n) {
        c = n;
        thr = 0;  // capture everything: the select then runs on the whole segment's copy
        thr_r = 0;
      } else {
        c = std::min(n, std::max(ks[s] * kCapacityFactor, kMinCapacity));
        thr_r = randk_threshold(n, ks[s]);
      }
      if (no_estimate) {
        thr = gc::kNoCapture;
        thr_r = gc::kNoCapture;
      }
    }
    if (ks[s] > 0) rk_scale[s] = (float)((double)n / (double)ks[s]);
    thr_rand[s] = thr_r;
    kk[s] = (uint32_t)ks[s];
    cap[s] = (uint32_t)c;
    thr_init[s] = thr;
    cand_base[s] = cand_total;
    cand_total += round_up(c, 4);
    chunk_base[s + 1] = chunk_base[s] + ceil_div(c, gc::kChunk);
    out_chunk_base[s + 1] = out_chunk_base[s] + ceil_div(ks[s], gc::kOutChunk);
  }
  const int64_t n_tiles = tile_base[n_seg], n_chunks = chunk_base[n_seg];
  // cold-start sample: about kSampleTiles evenly spaced tiles of each segment that starts
  // without an estimate (large segments with k > 0; none when the debug flags forbid one)
  std::vector<int32_t> sample_tile;
  std::vector<int64_t> sample_elems(n_seg, 0);
  if (!no_estimate) {
    for (int32_t s = 0; s < n_seg; ++s) {
      if (ks[s] == 0 || thr_init[s] != gc::kNoCapture || seg_flags[s]) continue;   // no estimate
      const int64_t nt = tile_base[s + 1] - tile_base[s];
      const int64_t stride = std::max<int64_t>(1, ceil_div(nt, kSampleTiles));
      for (int64_t j = 0; j < nt; j += stride) {
        sample_tile.push_back((int32_t)(tile_base[s] + j));
        sample_elems[s] += std::min<int64_t>(gc::kTile, seg_off[s + 1] - seg_off[s] - j * gc::kTile);
      }
    }
  }
  const int64_t n_sample = (int64_t)sample_tile.size();
  const int64_t n_out_chunks = out_chunk_base[n_seg];
  if (n_tiles > INT32_MAX || n_chunks + gc::kFullBlocks > INT32_MAX || n_out_chunks > INT32_MAX ||
      cand_total > UINT32_MAX * 4ll)
    return GC_ERR_UNSUPPORTED;
  std::vector<int32_t> tile_seg(n_tiles), chunk_seg(n_chunks), out_chunk_seg(n_out_chunks);
  std::vector<int4> tile_desc(n_tiles);
  for (int32_t s = 0; s < n_seg; ++s) {
    for (int64_t t = tile_base[s]; t < tile_base[s + 1]; ++t) {
      tile_seg[t] = s;
      const int64_t start = seg_off[s] + (t - tile_base[s]) * gc::kTile;
      const int64_t len = std::min<int64_t>(gc::kTile, seg_off[s + 1] - start);
      tile_desc[t] = make_int4((int)(uint32_t)start, (int)(uint32_t)((uint64_t)start >> 32),
                               (int)len, s);
    }
    for (int64_t c = chunk_base[s]; c < chunk_base[s + 1]; ++c) chunk_seg[c] = s;
    for (int64_t c = out_chunk_base[s]; c < out_chunk_base[s + 1]; ++c) out_chunk_seg[c] = s;
  }

  // device workspace
  gc::DevPlan& d = p->dp;
  d.n_seg = n_seg;
  d.flags = (int32_t)flags;
  d.n_tiles = n_tiles;
  d.n_chunks = n_chunks;
  d.n_chunk_blocks = gc::chunk_walkers(n_chunks);
  d.single = (flags & GC_DEBUG_CHAIN) ? 0 : 1;
  for (int32_t s = 0; s < n_seg && d.single; ++s)
    if (!gc::single_segment_ok(seg_off[s + 1] - seg_off[s], ks[s])) d.single = 0;
  int64_t *d_seg_off, *d_tile_base, *d_chunk_base, *d_out_off, *d_cand_base, *d_out_chunk_base;
  int32_t *d_tile_seg, *d_chunk_seg, *d_out_chunk_seg;
  int4* d_tile_desc;
  uint32_t *d_k, *d_cap, *d_thr_init;
  Carver cv;
  cv.add(&d_seg_off, n_seg + 1);
  cv.add(&d_tile_base, n_seg + 1);
  cv.add(&d_tile_seg, n_tiles);
  cv.add(&d_tile_desc, n_tiles);
  cv.add(&d_chunk_base, n_seg + 1);
  cv.add(&d_chunk_seg, n_chunks);
  cv.add(&d_k, n_seg);
  cv.add(&d_out_off, n_seg + 1);
  cv.add(&d_cand_base, n_seg);
  cv.add(&d_cap, n_seg);
  cv.add(&d_thr_init, n_seg);
  cv.add(&d_out_chunk_seg, n_out_chunks);
  cv.add(&d_out_chunk_base, n_seg + 1);
  uint32_t* d_seg_flags;
  cv.add(&d_seg_flags, n_seg);
  cv.add(&d.thr, n_seg);
  cv.add(&d.cand_cnt, n_seg);
  cv.add(&d.recap_cnt, n_seg);
  cv.add(&d.mode, n_seg);
  cv.add(&d.thr_lo, n_seg);
  cv.add(&d.pfx1, n_seg);
  cv.add(&d.kk1, n_seg);
  cv.add(&d.pfx2, n_seg);
  cv.add(&d.kk2, n_seg);
  cv.add(&d.kth, n_seg);
  cv.add(&d.ties, n_seg);
  cv.add(&d.sel_cnt, n_seg);
  cv.add(&d.hist, (int64_t)n_seg * 3 * gc::kHistBins);
  cv.add(&d.full_list, n_seg);
  cv.add(&d.full_count, 1);
  cv.add(&d.pend_list, n_seg);
  cv.add(&d.pend_count, 1);
  cv.add(&d.near_cnt, n_seg);
  cv.add(&d.beta, n_seg);
  cv.add(&d.err, 1);

  cv.add(&d.run_off, n_tiles);
  cv.add(&d.run_cnt, n_tiles);
  cv.add(&d.run_dst, n_tiles);
  cv.add(&d.tile_gt, n_tiles);
  cv.add(&d.tile_eq, n_tiles);
  cv.add(&d.tile_eq_base, n_tiles);
  cv.add(&d.tile_sel_base, n_tiles);
  cv.add(&d.chunk_gt, n_chunks);
  cv.add(&d.chunk_max, n_chunks);
  cv.add(&d.chunk_eq, n_chunks);
  cv.add(&d.chunk_eq_base, n_chunks);
  cv.add(&d.chunk_sel_base, n_chunks);
  cv.add(&d.act_chunk, n_chunks);
  cv.add(&d.act_count, 1);
  cv.add(&d.tile_max, n_tiles);
  cv.add(&d.tile_l1, n_tiles);
  int64_t* d_word_off;
  cv.add(&d_word_off, n_seg + 1);
  cv.add(&d.cand_val, cand_total);
  cv.add(&d.cand_idx, cand_total);
  cv.add(&d.sort_val, cand_total);
  cv.add(&d.sort_idx, cand_total);
  uint32_t* d_thr_rand;
  float* d_rk_scale;
  cv.add(&d.seg_norm, n_seg);
  int32_t* d_sample_tile;
  int64_t* d_sample_elems;
  cv.add(&d_sample_tile, n_sample);
  cv.add(&d_sample_elems, n_seg);
  cv.add(&d.thr_est, n_seg);
  cv.add(&d.beta_est, n_seg);
  cv.add(&d.tau_cnt, n_seg);
  cv.add(&d_thr_rand, n_seg);
  cv.add(&d_rk_scale, n_seg);
  const std::vector<float> beta_init(n_seg, gc::kInitialBeta);
  const std::vector<uint32_t> no_floor(n_seg, gc::kNoCapture);
  if (hipMalloc(&p->mem, cv.total()) != hipSuccess) {
    (void)hipGetLastError();
    return GC_ERR_OOM;
  }
  cv.place(static_cast<char*>(p->mem));
  d.seg_off = d_seg_off;
  d.tile_base = d_tile_base;
  d.tile_seg = d_tile_seg;
  d.tile_desc = d_tile_desc;
  d.chunk_base = d_chunk_base;
  d.chunk_seg = d_chunk_seg;
  d.k = d_k;
  d.out_off = d_out_off;
  d.cand_base = d_cand_base;
  d.cand_cap = d_cap;
  d.thr_init = d_thr_init;
  d.seg_flags = d_seg_flags;
  d.codec = gc::kCodecTopk;
  d.word_off = d_word_off;
  d.thr_rand = d_thr_rand;
  d.rk_scale = d_rk_scale;
  d.keys = gc::kKeysMagnitude;
  d.n_sample = n_sample;
  d.sample_tile = d_sample_tile;
  d.sample_elems = d_sample_elems;
  gc::OutPlan& o = p->op;
  o.n_seg = n_seg;
  o.n_out_chunks = n_out_chunks;
  o.seg_off = d_seg_off;
  o.out_off = d_out_off;
  o.out_chunk_seg = d_out_chunk_seg;
  o.out_chunk_base = d_out_chunk_base;

  hipError_t err = hipSuccess;
  auto up = [&](hipError_t e) { if (err == hipSuccess) err = e; };
  up(upload(d_seg_off, p->seg_off));
  up(upload(d_tile_base, tile_base));
  up(upload(d_tile_seg, tile_seg));
  up(upload(d_tile_desc, tile_desc));
  up(upload(d_chunk_base, chunk_base));
  up(upload(d_chunk_seg, chunk_seg));
  up(upload(d_k, kk));
  up(upload(d_out_off, p->out_off));
  up(upload(d_cand_base, cand_base));
  up(upload(d_cap, cap));
  up(upload(d_thr_init, thr_init));
  up(upload(d_seg_flags, seg_flags));
  up(upload(d_out_chunk_seg, out_chunk_seg));
  up(upload(d_out_chunk_base, out_chunk_base));
  up(upload(d_word_off, p->word_off));
  up(upload(d_thr_rand, thr_rand));
  up(upload(d_rk_scale, rk_scale));
  up(upload(d_sample_tile, sample_tile));
  up(upload(d_sample_elems, sample_elems));
  up(upload(d.thr, thr_init));
  up(upload(d.beta, beta_init));
  up(upload(d.thr_est, no_floor));
  up(upload(d.beta_est, beta_init));
  // the per-call counters and histograms start at zero (each call clears what it used)
  const size_t seg_bytes = sizeof(uint32_t) * std::max(n_seg, 1);
  for (uint32_t* a : {d.cand_cnt, d.recap_cnt, d.tau_cnt, d.near_cnt, d.mode, d.kth, d.ties,
                      d.sel_cnt})
    up(hipMemset(a, 0, seg_bytes));
  up(hipMemset(d.pend_count, 0, sizeof(uint32_t)));
  up(hipMemset(d.hist, 0, sizeof(uint32_t) * std::max<int64_t>((int64_t)n_seg * 3 * gc::kHistBins, 1)));
  up(hipMemset(d.err, 0, sizeof(uint32_t)));
  up(hipMemset(d.act_count, 0, sizeof(uint32_t)));
  up(hipMemset(d.full_count, 0, sizeof(uint32_t)));
  up(hipDeviceSynchronize());
  if (err != hipSuccess) {
    (void)hipGetLastError();
    (void)hipFree(p->mem);
    return GC_ERR_HIP;
  }
  *out = p.release();
  return GC_OK;
}

}  // namespace

extern "C" {

int gc_plan_create(const int64_t* seg_off, int32_t n_seg, const int64_t* k, const double* ratio,
                   uint32_t flags, gc_plan** out) {
  if (!out) return GC_ERR_INVALID_ARG;
  *out = nullptr;
  if (n_seg < 0 || !seg_off) return GC_ERR_INVALID_ARG;
  if (flags & ~(uint32_t)(GC_MOMENTUM_MASK | GC_DEBUG_FORCE_FALLBACK | GC_DEBUG_NO_ESTIMATE |
                          GC_DEBUG_CHAIN))
    return GC_ERR_INVALID_ARG;
  try {
    return plan_create(seg_off, n_seg, k, ratio, flags, out);
  } catch (const std::bad_alloc&) {
    return GC_ERR_OOM;
  }
}

int gc_plan_destroy(gc_plan* plan) {
  if (!plan) return GC_OK;
  int rc = GC_OK;
  int cur = -1;
  const bool switched = hipGetDevice(&cur) == hipSuccess && cur != plan->device &&
                        hipSetDevice(plan->device) == hipSuccess;
  if (hipDeviceSynchronize() != hipSuccess) rc = GC_ERR_HIP;
  for (auto& pr : plan->pending) {
    (void)hipEventDestroy(pr.first);
    (void)hipEventDestroy(pr.second);
  }
  for (auto& pr : plan->spare) {
    (void)hipEventDestroy(pr.first);
    (void)hipEventDestroy(pr.second);
  }
  if (plan->mem && hipFree(plan->mem) != hipSuccess) rc = GC_ERR_HIP;
  if (switched) (void)hipSetDevice(cur);
  delete plan;
  return rc;
}

int gc_plan_total_k(const gc_plan* plan, int64_t* total_k) {
  if (!plan || !total_k) return GC_ERR_INVALID_ARG;
  *total_k = plan->total_k;
  return GC_OK;
}

int gc_plan_layout(const gc_plan* plan, int64_t* k, int64_t* out_off) {
  if (!plan) return GC_ERR_INVALID_ARG;
  if (k && plan->n_seg) std::memcpy(k, plan->k.data(), sizeof(int64_t) * plan->n_seg);
  if (out_off) std::memcpy(out_off, plan->out_off.data(), sizeof(int64_t) * (plan->n_seg + 1));
  return GC_OK;
}

}  // extern "C"

namespace {
// With timing on, a HIP event pair for the streaming passes of this call.
int timing_events(gc_plan* plan, hipEvent_t* b, hipEvent_t* en) {
  if (!plan->timing) return GC_OK;
  try {  // room for the pair in both lists, so nothing below can throw
    plan->pending.reserve(plan->pending.size() + 1);
    plan->spare.reserve(plan->spare.size() + plan->pending.size() + 1);
  } catch (const std::bad_alloc&) {
    return GC_ERR_OOM;
  }
  if (plan->spare.empty()) {
    hipEvent_t x, y;
    if (hipEventCreate(&x) != hipSuccess) return GC_ERR_HIP;
    if (hipEventCreate(&y) != hipSuccess) {
      (void)hipEventDestroy(x);
      return GC_ERR_HIP;
    }
    plan->spare.emplace_back(x, y);
  }
  *b = plan->spare.back().first;
  *en = plan->spare.back().second;
  plan->pending.push_back(plan->spare.back());
  plan->spare.pop_back();
  return GC_OK;
}

int compress_checked(gc_plan* plan, const float* g, float* e, float* u, float momentum,
                     float* out_vals, int32_t* out_idx, const gc::Int8Args& q8, void* stream) {
  if (!plan) return GC_ERR_INVALID_ARG;
  const bool any = plan->seg_off[plan->n_seg] > plan->seg_off[0];
  if (any && (!g || !e || !aligned16(g) || !aligned16(e))) return GC_ERR_INVALID_ARG;
  if (u && !aligned16(u)) return GC_ERR_INVALID_ARG;
  if (plan->total_k > 0 && !out_idx) return GC_ERR_INVALID_ARG;
  const int64_t kt = plan->total_k;
  if (any_overlap({dense_span(plan, g, 4), dense_span(plan, e, 4), dense_span(plan, u, 4), flat(out_vals, kt, 4),
                   flat(out_idx, kt, 4), flat(q8.codes, kt, 1), flat(q8.scales, plan->n_seg, 4)}))
    return GC_ERR_INVALID_ARG;
  if (int rc = check_device(plan)) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipEvent_t b = nullptr, en = nullptr;
  if (int rc = timing_events(plan, &b, &en)) return rc;
  const hipError_t err = gc::launch_compress(plan->dp, g, e, u, momentum, out_vals, out_idx,
                                             q8, plan->cold, st, b, en);
  plan->cold = false;
  return err == hipSuccess ? GC_OK : GC_ERR_HIP;
}

}  // namespace

extern "C" {

int gc_topk_ef_compress(gc_plan* plan, const float* g, float* e, float* u, float momentum,
                        float* out_vals, int32_t* out_idx, void* stream) {
  if (plan && plan->total_k > 0 && !out_vals) return GC_ERR_INVALID_ARG;
  return compress_checked(plan, g, e, u, momentum, out_vals, out_idx, gc::Int8Args{}, stream);
}

int gc_topk_ef_compress_int8(gc_plan* plan, const float* g, float* e, float* u, float momentum,
                             uint64_t seed, uint64_t step, float* out_vals, int32_t* out_idx,
                             int8_t* out_codes, float* out_scales, void* stream) {
  if (!plan) return GC_ERR_INVALID_ARG;
  if ((plan->total_k > 0 && !out_codes) || (plan->n_seg > 0 && !out_scales))
    return GC_ERR_INVALID_ARG;
  gc::Int8Args q8{};
  q8.enabled = 1;
  q8.codes = out_codes;
  q8.scales = out_scales;
  q8.seed_lo = (uint32_t)seed;
  q8.seed_hi = (uint32_t)(seed >> 32);
  q8.step_lo = (uint32_t)step;
  if (plan->n_seg == 0) return GC_OK;
  return compress_checked(plan, g, e, u, momentum, out_vals, out_idx, q8, stream);
}

int gc_threshold_ef_compress(gc_plan* plan, const float* g, float* e, float* u, float momentum,
                             const float* tau, float* out_vals, int32_t* out_idx,
                             int32_t* out_count, void* stream) {
  if (!plan) return GC_ERR_INVALID_ARG;
  const bool any = plan->seg_off[plan->n_seg] > plan->seg_off[0];
  if (any && (!g || !e || !aligned16(g) || !aligned16(e))) return GC_ERR_INVALID_ARG;
  if (u && !aligned16(u)) return GC_ERR_INVALID_ARG;
  if (plan->n_seg > 0 && !tau) return GC_ERR_INVALID_ARG;
  if (plan->total_k > 0 && (!out_vals || !out_idx)) return GC_ERR_INVALID_ARG;
  const int64_t kt = plan->total_k, ns = plan->n_seg;
  if (any_overlap({dense_span(plan, g, 4), dense_span(plan, e, 4), dense_span(plan, u, 4), flat(tau, ns, 4),
                   flat(out_vals, kt, 4), flat(out_idx, kt, 4), flat(out_count, ns, 4)}))
    return GC_ERR_INVALID_ARG;
  if (int rc = check_device(plan)) return rc;
  hipEvent_t b = nullptr, en = nullptr;
  if (int rc = timing_events(plan, &b, &en)) return rc;
  const hipError_t err =
      gc::launch_threshold(plan->dp, g, e, u, momentum, tau, out_vals, out_idx,
                           out_count, static_cast<hipStream_t>(stream), b, en);
  return err == hipSuccess ? GC_OK : GC_ERR_HIP;
}

int gc_randk_compress(gc_plan* plan, const float* g, float* e, float* u, float momentum,
                      uint64_t seed, uint64_t step, float* out_vals, int32_t* out_idx,
                      void* stream) {
  if (!plan) return GC_ERR_INVALID_ARG;
  const bool any = plan->seg_off[plan->n_seg] > plan->seg_off[0];
  if (any && (!g || !aligned16(g))) return GC_ERR_INVALID_ARG;
  if ((e && !aligned16(e)) || (u && !aligned16(u))) return GC_ERR_INVALID_ARG;
  if (plan->total_k > 0 && (!out_vals || !out_idx)) return GC_ERR_INVALID_ARG;
  const int64_t kt = plan->total_k;
  if (any_overlap({dense_span(plan, g, 4), dense_span(plan, e, 4), dense_span(plan, u, 4), flat(out_vals, kt, 4),
                   flat(out_idx, kt, 4)}))
    return GC_ERR_INVALID_ARG;
  if (int rc = check_device(plan)) return rc;
  hipEvent_t b = nullptr, en = nullptr;
  if (int rc = timing_events(plan, &b, &en)) return rc;
  const hipError_t err = gc::launch_randk(plan->dp, g, e, u, momentum, seed, step, out_vals,
                                          out_idx, static_cast<hipStream_t>(stream), b, en);
  return err == hipSuccess ? GC_OK : GC_ERR_HIP;
}

int gc_plan_sign_layout(const gc_plan* plan, int64_t* word_off) {
  if (!plan || !word_off) return GC_ERR_INVALID_ARG;
  std::memcpy(word_off, plan->word_off.data(), sizeof(int64_t) * (plan->n_seg + 1));
  return GC_OK;
}

int gc_sign_ef_compress(gc_plan* plan, const float* g, float* e, float* u, float momentum,
                        uint32_t* out_bits, float* out_scales, void* stream) {
  if (!plan) return GC_ERR_INVALID_ARG;
  const bool any = plan->seg_off[plan->n_seg] > plan->seg_off[0];
  if (any && (!g || !e || !out_bits || !aligned16(g) || !aligned16(e))) return GC_ERR_INVALID_ARG;
  if (u && !aligned16(u)) return GC_ERR_INVALID_ARG;
  if (plan->n_seg > 0 && !out_scales) return GC_ERR_INVALID_ARG;
  if (any_overlap({dense_span(plan, g, 4), dense_span(plan, e, 4), dense_span(plan, u, 4),
                   flat(out_bits, plan->word_off[plan->n_seg], 4),
                   flat(out_scales, plan->n_seg, 4)}))
    return GC_ERR_INVALID_ARG;
  if (int rc = check_device(plan)) return rc;
  hipEvent_t b = nullptr, en = nullptr;
  if (int rc = timing_events(plan, &b, &en)) return rc;
  const hipError_t err = gc::launch_sign(plan->dp, g, e, u, momentum, out_bits, out_scales,
                                         static_cast<hipStream_t>(stream), b, en);
  return err == hipSuccess ? GC_OK : GC_ERR_HIP;
}

int gc_sign_decompress(const gc_plan* plan, const uint32_t* bits, const float* scales,
                       float* dense, int accumulate, void* stream) {
  if (!plan) return GC_ERR_INVALID_ARG;
  const bool any = plan->seg_off[plan->n_seg] > plan->seg_off[0];
  if (any && (!bits || !scales || !dense)) return GC_ERR_INVALID_ARG;
  if (any_overlap({dense_span(plan, dense, 4), flat(bits, plan->word_off[plan->n_seg], 4),
                   flat(scales, plan->n_seg, 4)}))
    return GC_ERR_INVALID_ARG;
  if (int rc = check_device(plan)) return rc;
  const hipError_t err = gc::launch_sign_decompress(plan->dp, bits, scales, dense, accumulate,
                                                    static_cast<hipStream_t>(stream));
  return err == hipSuccess ? GC_OK : GC_ERR_HIP;
}

int gc_qsgd_compress(gc_plan* plan, const float* g, float* e, float* u, float momentum,
                     int32_t levels, uint64_t seed, uint64_t step, int8_t* out_codes,
                     float* out_norms, void* stream) {
  if (!plan || levels < 1 || levels > 127) return GC_ERR_INVALID_ARG;
  const bool any = plan->seg_off[plan->n_seg] > plan->seg_off[0];
  if (any && (!g || !out_codes || !aligned16(g) || (reinterpret_cast<uintptr_t>(out_codes) & 3)))
    return GC_ERR_INVALID_ARG;
  if ((e && !aligned16(e)) || (u && !aligned16(u))) return GC_ERR_INVALID_ARG;
  if (plan->n_seg > 0 && !out_norms) return GC_ERR_INVALID_ARG;
  if (any_overlap({dense_span(plan, g, 4), dense_span(plan, e, 4), dense_span(plan, u, 4),
                   dense_span(plan, out_codes, 1), flat(out_norms, plan->n_seg, 4)}))
    return GC_ERR_INVALID_ARG;
  if (int rc = check_device(plan)) return rc;
  hipEvent_t b = nullptr, en = nullptr;
  if (int rc = timing_events(plan, &b, &en)) return rc;
  const hipError_t err = gc::launch_qsgd(plan->dp, g, e, u, momentum, levels, seed, step,
                                         out_codes, out_norms, static_cast<hipStream_t>(stream),
                                         b, en);
  return err == hipSuccess ? GC_OK : GC_ERR_HIP;
}

int gc_qsgd_decompress(const gc_plan* plan, const int8_t* codes, const float* norms,
                       int32_t levels, float* dense, int accumulate, void* stream) {
  if (!plan || levels < 1 || levels > 127) return GC_ERR_INVALID_ARG;
  const bool any = plan->seg_off[plan->n_seg] > plan->seg_off[0];
  if (any && (!codes || !norms || !dense)) return GC_ERR_INVALID_ARG;
  if (any_overlap({dense_span(plan, dense, 4), dense_span(plan, codes, 1), flat(norms, plan->n_seg, 4)}))
    return GC_ERR_INVALID_ARG;
  if (int rc = check_device(plan)) return rc;
  const hipError_t err = gc::launch_qsgd_decompress(plan->dp, codes, norms, levels, dense,
                                                    accumulate, static_cast<hipStream_t>(stream));
  return err == hipSuccess ? GC_OK : GC_ERR_HIP;
}

int gc_quant_int8(gc_plan* plan, const float* vals, const int32_t* idx, float* e, uint64_t seed,
                  uint64_t step, int8_t* out_codes, float* out_scales, void* stream) {
  if (!plan) return GC_ERR_INVALID_ARG;
  if (plan->total_k > 0 && (!vals || !idx || !out_codes)) return GC_ERR_INVALID_ARG;
  if (plan->n_seg > 0 && !out_scales) return GC_ERR_INVALID_ARG;
  const int64_t kt = plan->total_k;
  if (any_overlap({flat(vals, kt, 4), flat(idx, kt, 4), dense_span(plan, e, 4), flat(out_codes, kt, 1),
                   flat(out_scales, plan->n_seg, 4)}))
    return GC_ERR_INVALID_ARG;
  if (int rc = check_device(plan)) return rc;
  const hipError_t err = gc::launch_quant(plan->op, vals, idx, e, seed, step, out_codes,
                                          out_scales, static_cast<hipStream_t>(stream));
  return err == hipSuccess ? GC_OK : GC_ERR_HIP;
}

int gc_decompress(const gc_plan* plan, const float* vals, const int8_t* codes,
                  const float* scales, const int32_t* idx, float* dense, int accumulate,
                  void* stream) {
  if (!plan) return GC_ERR_INVALID_ARG;
  if ((vals == nullptr) == (codes == nullptr)) return GC_ERR_INVALID_ARG;
  if (codes && !scales) return GC_ERR_INVALID_ARG;
  if (plan->total_k > 0 && !idx) return GC_ERR_INVALID_ARG;
  if (!dense && plan->seg_off[plan->n_seg] > plan->seg_off[0]) return GC_ERR_INVALID_ARG;
  {
    const int64_t kt = plan->total_k;
    const Span out = dense_span(plan, dense, 4);
    if (any_overlap({out, flat(vals, kt, 4)}) || any_overlap({out, flat(codes, kt, 1)}) ||
        any_overlap({out, flat(scales, plan->n_seg, 4)}) || any_overlap({out, flat(idx, kt, 4)}))
      return GC_ERR_INVALID_ARG;
  }
  if (int rc = check_device(plan)) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t err = hipSuccess;
  if (!accumulate) err = gc::launch_fill_zero(dense, plan->seg_off[0], plan->seg_off[plan->n_seg], st);
  if (err == hipSuccess)
    err = gc::launch_decompress(plan->op, vals, codes, scales, idx, dense, accumulate, st);
  return err == hipSuccess ? GC_OK : GC_ERR_HIP;
}

int gc_decompress_gathered(const gc_plan* plan, int32_t n_workers, const float* vals,
                           const int8_t* codes, const float* scales, const int32_t* idx,
                           float* dense, int accumulate, void* stream) {
  if (!plan || n_workers < 0) return GC_ERR_INVALID_ARG;
  if ((vals == nullptr) == (codes == nullptr)) return GC_ERR_INVALID_ARG;
  if (codes && !scales) return GC_ERR_INVALID_ARG;
  if (plan->total_k > 0 && n_workers > 0 && !idx) return GC_ERR_INVALID_ARG;
  if (!dense && plan->seg_off[plan->n_seg] > plan->seg_off[0]) return GC_ERR_INVALID_ARG;
  {
    const int64_t wk = (int64_t)n_workers * plan->total_k;
    const Span out = dense_span(plan, dense, 4);
    if (any_overlap({out, flat(vals, wk, 4)}) || any_overlap({out, flat(codes, wk, 1)}) ||
        any_overlap({out, flat(scales, (int64_t)n_workers * plan->n_seg, 4)}) ||
        any_overlap({out, flat(idx, wk, 4)}))
      return GC_ERR_INVALID_ARG;
  }
  if (int rc = check_device(plan)) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t err = hipSuccess;
  if (!accumulate) err = gc::launch_fill_zero(dense, plan->seg_off[0], plan->seg_off[plan->n_seg], st);
  const int64_t kk = plan->total_k;
  // one ordered pass per worker: the additions into each position happen in worker order
  for (int32_t w = 0; w < n_workers && err == hipSuccess; ++w)
    err = gc::launch_decompress(plan->op, vals ? vals + (int64_t)w * kk : nullptr,
                                codes ? codes + (int64_t)w * kk : nullptr,
                                scales ? scales + (int64_t)w * plan->n_seg : nullptr,
                                idx + (int64_t)w * kk, dense, 1, st);
  return err == hipSuccess ? GC_OK : GC_ERR_HIP;
}

int gc_clip_by_norm(gc_plan* plan, float* g, const float* max_norm, float* norms_out,
                    void* stream) {
  if (!plan) return GC_ERR_INVALID_ARG;
  const bool any = plan->seg_off[plan->n_seg] > plan->seg_off[0];
  if (any && (!g || !aligned16(g))) return GC_ERR_INVALID_ARG;
  if (plan->n_seg > 0 && !max_norm) return GC_ERR_INVALID_ARG;
  if (any_overlap({dense_span(plan, g, 4), flat(max_norm, plan->n_seg, 4),
                   flat(norms_out, plan->n_seg, 4)}))
    return GC_ERR_INVALID_ARG;
  if (int rc = check_device(plan)) return rc;
  const hipError_t err = gc::launch_clip(plan->dp, g, max_norm,
                                         norms_out ? norms_out : plan->dp.seg_norm, nullptr,
                                         static_cast<hipStream_t>(stream));
  return err == hipSuccess ? GC_OK : GC_ERR_HIP;
}

int gc_clip_factors(gc_plan* plan, const float* g, const float* max_norm, float* norms_out,
                    float* factors_out, void* stream) {
  if (!plan) return GC_ERR_INVALID_ARG;
  const bool any = plan->seg_off[plan->n_seg] > plan->seg_off[0];
  if (any && (!g || !aligned16(g))) return GC_ERR_INVALID_ARG;
  if (plan->n_seg > 0 && (!max_norm || !factors_out)) return GC_ERR_INVALID_ARG;
  if (any_overlap({dense_span(plan, g, 4), flat(max_norm, plan->n_seg, 4),
                   flat(norms_out, plan->n_seg, 4), flat(factors_out, plan->n_seg, 4)}))
    return GC_ERR_INVALID_ARG;
  if (int rc = check_device(plan)) return rc;
  const hipError_t err = gc::launch_clip(plan->dp, const_cast<float*>(g), max_norm,
                                         norms_out ? norms_out : plan->dp.seg_norm, factors_out,
                                         static_cast<hipStream_t>(stream));
  return err == hipSuccess ? GC_OK : GC_ERR_HIP;
}

int gc_plan_set_gradient_scale(gc_plan* plan, const float* factors) {
  if (!plan) return GC_ERR_INVALID_ARG;
  plan->dp.gscale = factors;
  return GC_OK;
}

int gc_plan_reset_estimate(gc_plan* plan, void* stream) {
  if (!plan) return GC_ERR_INVALID_ARG;
  if (int rc = check_device(plan)) return rc;
  plan->cold = true;
  return gc::launch_reset(plan->dp, static_cast<hipStream_t>(stream)) == hipSuccess ? GC_OK
                                                                                     : GC_ERR_HIP;
}

int gc_plan_last_stats(gc_plan* plan, uint32_t* mode, uint32_t* candidates, uint32_t* kth_key,
                       uint32_t* ties_taken, void* stream) {
  if (!plan) return GC_ERR_INVALID_ARG;
  if (int rc = check_device(plan)) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const size_t bytes = sizeof(uint32_t) * plan->n_seg;
  hipError_t err = hipSuccess;
  auto cp = [&](uint32_t* dst, const uint32_t* src) {
    if (dst && bytes && err == hipSuccess) err = hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToHost, st);
  };
  cp(mode, plan->dp.mode);
  cp(candidates, plan->dp.sel_cnt);
  cp(kth_key, plan->dp.kth);
  cp(ties_taken, plan->dp.ties);
  uint32_t flag = 0;
  if (err == hipSuccess) err = hipMemcpyAsync(&flag, plan->dp.err, sizeof flag, hipMemcpyDeviceToHost, st);
  if (err == hipSuccess) err = hipStreamSynchronize(st);
  if (err != hipSuccess) return GC_ERR_HIP;
  return flag ? GC_ERR_HIP : GC_OK;
}

int gc_plan_set_timing(gc_plan* plan, int enable) {
  if (!plan) return GC_ERR_INVALID_ARG;
  plan->timing = enable != 0;
  return GC_OK;
}

int gc_plan_timing(gc_plan* plan, double* ms, int64_t* launches) {
  if (!plan || !ms || !launches) return GC_ERR_INVALID_ARG;
  double sum = 0.0;
  int64_t n = 0;
  int rc = GC_OK;
  for (auto& pr : plan->pending) {
    float t = 0.0f;
    if (hipEventSynchronize(pr.second) != hipSuccess ||
        hipEventElapsedTime(&t, pr.first, pr.second) != hipSuccess)
      rc = GC_ERR_HIP;
    sum += t;
    ++n;
    plan->spare.push_back(pr);
  }
  plan->pending.clear();
  *ms = sum;
  *launches = n;
  return rc;
}

int gc_copy_f32(const float* src, float* dst, int64_t n, void* stream) {
  if (n < 0 || (n & 3) || (n && (!src || !dst || !aligned16(src) || !aligned16(dst))))
    return GC_ERR_INVALID_ARG;
  return gc::launch_copy(src, dst, n, static_cast<hipStream_t>(stream)) == hipSuccess ? GC_OK
                                                                                      : GC_ERR_HIP;
}

int gc_add_f32(const float* x, float* y, int64_t n, void* stream) {
  if (n < 0 || (n && (!x || !y || !aligned16(x) || !aligned16(y)))) return GC_ERR_INVALID_ARG;
  if (any_overlap({flat(x, n, 4), flat(y, n, 4)})) return GC_ERR_INVALID_ARG;
  return gc::launch_add(x, y, n, static_cast<hipStream_t>(stream)) == hipSuccess ? GC_OK
                                                                                 : GC_ERR_HIP;
}

}  // extern "C"

// ------------------------------------------------------------------------------------------
// The entry point that allocates nothing (gc_topk_ef_compress_noalloc).  Its plan lives in
// `scratch`, a file-scope device array: the segment table, the tile and chunk tables, the
// per-segment and per-tile state, the histograms and the candidate buffers of one call, for
// at most GC_NOALLOC_MAX_SEGMENTS segments and GC_NOALLOC_MAX_ELEMENTS elements.  A setup
// kernel writes the tables and clears the state at the start of every call (no host table is
// built, no memory is allocated, no memset is recorded), then the call runs the same kernels
// as gc_topk_ef_compress, without a threshold estimate (every segment takes the exact
// re-capture or full path).  Every call on a device shares that device's array: calls that
// overlap on one device race.
namespace {

constexpr int kNaSeg = GC_NOALLOC_MAX_SEGMENTS;
constexpr int64_t kNaElems = GC_NOALLOC_MAX_ELEMENTS;
constexpr int64_t kNaCand = GC_NOALLOC_MAX_CANDIDATES;
constexpr int64_t kNaTiles = kNaElems / gc::kTile + kNaSeg;         // ragged tail per segment
constexpr int64_t kNaCandSlots = kNaCand + 4 * kNaSeg;              // each region rounded up to 4
constexpr int64_t kNaChunks = kNaCandSlots / gc::kChunk + kNaSeg;
constexpr size_t kScratchBytes = (size_t)24 << 20;
constexpr int kNaMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_na_mu;
void* g_na_ptr[kNaMaxDevices];   // the device address of `scratch` on each device

// Segment table of one call, passed to the setup kernel by value.
struct NaArgs {
  int32_t n_seg;
  int32_t flags;
  int64_t seg_off[kNaSeg + 1];
  int64_t k[kNaSeg];
  int64_t cap[kNaSeg];
};

// Candidate capacity of a segment in the static array (the results never depend on it: a
// bucket larger than the capacity takes the exact full-segment path).
inline int64_t na_capacity(int64_t n, int64_t k) {
  if (k == 0 || n <= gc::kSmallSegment) return 0;   // small segments are selected whole
  return std::min(n, std::max(k * 4, (int64_t)65536));
}

// Sequential 256-byte-aligned pieces of the static array.
struct NaCarve {
  char* base;
  size_t off = 0;
  template <typename T>
  T* take(int64_t count) {
    off = (off + 255) & ~(size_t)255;
    T* p = reinterpret_cast<T*>(base + off);
    off += (size_t)std::max<int64_t>(count, 1) * sizeof(T);
    return p;
  }
};

// The plan of a call inside the static array (host arithmetic on the device address only).
size_t na_layout(char* base, gc::DevPlan& d) {
  NaCarve c{base};
  d.seg_off = c.take<int64_t>(kNaSeg + 1);
  d.tile_base = c.take<int64_t>(kNaSeg + 1);
  d.chunk_base = c.take<int64_t>(kNaSeg + 1);
  d.out_off = c.take<int64_t>(kNaSeg + 1);
  d.cand_base = c.take<int64_t>(kNaSeg);
  d.word_off = c.take<int64_t>(kNaSeg + 1);
  d.sample_elems = c.take<int64_t>(kNaSeg);
  d.k = c.take<uint32_t>(kNaSeg);
  d.cand_cap = c.take<uint32_t>(kNaSeg);
  d.thr_init = c.take<uint32_t>(kNaSeg);
  d.seg_flags = c.take<uint32_t>(kNaSeg);
  d.thr_rand = c.take<uint32_t>(kNaSeg);
  d.rk_scale = c.take<float>(kNaSeg);
  d.thr = c.take<uint32_t>(kNaSeg);
  d.cand_cnt = c.take<uint32_t>(kNaSeg);
  d.recap_cnt = c.take<uint32_t>(kNaSeg);
  d.mode = c.take<uint32_t>(kNaSeg);
  d.thr_lo = c.take<uint32_t>(kNaSeg);
  d.pfx1 = c.take<uint32_t>(kNaSeg);
  d.kk1 = c.take<uint32_t>(kNaSeg);
  d.pfx2 = c.take<uint32_t>(kNaSeg);
  d.kk2 = c.take<uint32_t>(kNaSeg);
  d.kth = c.take<uint32_t>(kNaSeg);
  d.ties = c.take<uint32_t>(kNaSeg);
  d.sel_cnt = c.take<uint32_t>(kNaSeg);
  d.beta = c.take<float>(kNaSeg);
  d.full_list = c.take<uint32_t>(kNaSeg);
  d.pend_list = c.take<uint32_t>(kNaSeg);
  d.near_cnt = c.take<uint32_t>(kNaSeg);
  d.thr_est = c.take<uint32_t>(kNaSeg);
  d.beta_est = c.take<float>(kNaSeg);
  d.tau_cnt = c.take<uint32_t>(kNaSeg);
  d.seg_norm = c.take<float>(kNaSeg);
  d.full_count = c.take<uint32_t>(1);
  d.pend_count = c.take<uint32_t>(1);
  d.act_count = c.take<uint32_t>(1);
  d.err = c.take<uint32_t>(1);
  d.hist = c.take<uint32_t>((int64_t)kNaSeg * 3 * gc::kHistBins);
  d.tile_seg = c.take<int32_t>(kNaTiles);
  d.tile_desc = c.take<int4>(kNaTiles);
  d.run_off = c.take<uint32_t>(kNaTiles);
  d.run_cnt = c.take<uint32_t>(kNaTiles);
  d.run_dst = c.take<uint32_t>(kNaTiles);
  d.tile_gt = c.take<uint32_t>(kNaTiles);
  d.tile_eq = c.take<uint32_t>(kNaTiles);
  d.tile_eq_base = c.take<uint32_t>(kNaTiles);
  d.tile_sel_base = c.take<uint32_t>(kNaTiles);
  d.tile_max = c.take<uint32_t>(kNaTiles);
  d.tile_l1 = c.take<double>(kNaTiles);
  d.chunk_seg = c.take<int32_t>(kNaChunks);
  d.chunk_gt = c.take<uint32_t>(kNaChunks);
  d.chunk_max = c.take<uint32_t>(kNaChunks);
  d.chunk_eq = c.take<uint32_t>(kNaChunks);
  d.chunk_eq_base = c.take<uint32_t>(kNaChunks);
  d.chunk_sel_base = c.take<uint32_t>(kNaChunks);
  d.act_chunk = c.take<uint32_t>(kNaChunks);
  d.cand_val = c.take<float>(kNaCandSlots);
  d.cand_idx = c.take<int32_t>(kNaCandSlots);
  d.sort_val = c.take<float>(kNaCandSlots);
  d.sort_idx = c.take<int32_t>(kNaCandSlots);
  return c.off;
}

// One workgroup: the per-segment tables (thread 0, at most kNaSeg segments), then the tile and
// chunk tables, and the per-call state cleared: no threshold (every segment takes the exact
// path), counters, flags and histograms zero.  It runs before every call, so nothing of the
// previous call (which may have had another segment table) is seen.
__global__ __launch_bounds__(1024) void k_noalloc_setup(gc::DevPlan P, NaArgs a) {
  __shared__ int64_t s_tile_base[kNaSeg + 1], s_chunk_base[kNaSeg + 1];
  if (threadIdx.x == 0) {
    int64_t tb = 0, cb = 0, ob = 0, kb = 0;
    for (int s = 0; s < a.n_seg; ++s) {
      const int64_t n = a.seg_off[s + 1] - a.seg_off[s];
      const_cast<int64_t*>(P.seg_off)[s] = a.seg_off[s];
      const_cast<int64_t*>(P.tile_base)[s] = tb;
      const_cast<int64_t*>(P.chunk_base)[s] = cb;
      const_cast<int64_t*>(P.out_off)[s] = ob;
      const_cast<int64_t*>(P.cand_base)[s] = kb;
      const_cast<int64_t*>(P.sample_elems)[s] = 0;
      const_cast<uint32_t*>(P.k)[s] = (uint32_t)a.k[s];
      const_cast<uint32_t*>(P.cand_cap)[s] = (uint32_t)a.cap[s];
      const_cast<uint32_t*>(P.thr_init)[s] = gc::kNoCapture;
      const_cast<uint32_t*>(P.seg_flags)[s] = n <= gc::kSmallSegment ? gc::kSegSmall : 0u;
      P.thr[s] = gc::kNoCapture;
      P.beta[s] = gc::kInitialBeta;
      P.cand_cnt[s] = 0;
      P.recap_cnt[s] = 0;
      P.tau_cnt[s] = 0;
      P.near_cnt[s] = 0;
      P.mode[s] = 0;
      P.kth[s] = 0;
      P.ties[s] = 0;
      P.sel_cnt[s] = 0;
      s_tile_base[s] = tb;
      s_chunk_base[s] = cb;
      tb += (n + gc::kTile - 1) / gc::kTile;
      cb += (a.cap[s] + gc::kChunk - 1) / gc::kChunk;
      ob += a.k[s];
      kb += (a.cap[s] + 3) / 4 * 4;
    }
    const_cast<int64_t*>(P.seg_off)[a.n_seg] = a.seg_off[a.n_seg];
    const_cast<int64_t*>(P.tile_base)[a.n_seg] = tb;
    const_cast<int64_t*>(P.chunk_base)[a.n_seg] = cb;
    const_cast<int64_t*>(P.out_off)[a.n_seg] = ob;
    s_tile_base[a.n_seg] = tb;
    s_chunk_base[a.n_seg] = cb;
    *P.full_count = 0;
    *P.pend_count = 0;
    *P.act_count = 0;
    *P.err = 0;
  }
  for (int64_t i = threadIdx.x; i < (int64_t)a.n_seg * 3 * gc::kHistBins; i += blockDim.x)
    P.hist[i] = 0;
  __syncthreads();
  for (int64_t t = threadIdx.x; t < s_tile_base[a.n_seg]; t += blockDim.x) {
    int s = 0;
    while (s_tile_base[s + 1] <= t) ++s;
    const int64_t start = a.seg_off[s] + (t - s_tile_base[s]) * gc::kTile;
    const int64_t len = std::min<int64_t>(gc::kTile, a.seg_off[s + 1] - start);
    const_cast<int32_t*>(P.tile_seg)[t] = s;
    const_cast<int4*>(P.tile_desc)[t] =
        make_int4((int)(uint32_t)start, (int)(uint32_t)((uint64_t)start >> 32), (int)len, s);
  }
  for (int64_t c = threadIdx.x; c < s_chunk_base[a.n_seg]; c += blockDim.x) {
    int s = 0;
    while (s_chunk_base[s + 1] <= c) ++s;
    const_cast<int32_t*>(P.chunk_seg)[c] = s;
  }
}

// The device address of `scratch` on the current device, looked up once per device.
int na_scratch(int dev, char** out) {
  if (dev < 0 || dev >= kNaMaxDevices) return GC_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_na_mu);
  if (!g_na_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return GC_ERR_HIP;
    }
    g_na_ptr[dev] = p;
  }
  *out = static_cast<char*>(g_na_ptr[dev]);
  return GC_OK;
}

}  // namespace

extern "C" {

int gc_topk_ef_compress_noalloc(const int64_t* seg_off, int32_t n_seg, const int64_t* k,
                                const double* ratio, uint32_t flags, const float* g, float* e,
                                float* u, float momentum, float* out_vals, int32_t* out_idx,
                                void* stream) {
  if (n_seg < 0 || !seg_off) return GC_ERR_INVALID_ARG;
  if (flags & ~(uint32_t)GC_MOMENTUM_MASK) return GC_ERR_INVALID_ARG;
  if (n_seg > kNaSeg) return GC_ERR_UNSUPPORTED;
  NaArgs a{};
  a.n_seg = n_seg;
  a.flags = (int32_t)flags;
  int64_t ks[kNaSeg > 0 ? kNaSeg : 1];
  if (int rc = gc_layout(seg_off, n_seg, k, ratio, ks, nullptr)) return rc;
  int64_t total_k = 0, cand = 0, tiles = 0, chunks = 0;
  for (int32_t s = 0; s < n_seg; ++s) {
    const int64_t n = seg_off[s + 1] - seg_off[s];
    a.seg_off[s] = seg_off[s];
    a.k[s] = ks[s];
    a.cap[s] = na_capacity(n, ks[s]);
    total_k += ks[s];
    cand += (a.cap[s] + 3) / 4 * 4;
    tiles += (n + gc::kTile - 1) / gc::kTile;
    chunks += (a.cap[s] + gc::kChunk - 1) / gc::kChunk;
  }
  a.seg_off[n_seg] = seg_off[n_seg];
  const int64_t n_all = seg_off[n_seg] - seg_off[0];
  if (n_all > kNaElems || cand > kNaCandSlots || tiles > kNaTiles || chunks > kNaChunks)
    return GC_ERR_UNSUPPORTED;
  if (n_all > 0 && (!g || !e || !aligned16(g) || !aligned16(e))) return GC_ERR_INVALID_ARG;
  if (u && !aligned16(u)) return GC_ERR_INVALID_ARG;
  if (total_k > 0 && (!out_vals || !out_idx)) return GC_ERR_INVALID_ARG;
  {
    const int64_t lo = seg_off[0];
    auto dspan = [&](const void* p) -> Span {
      if (!p) return {nullptr, 0};
      return {static_cast<const char*>(p) + lo * 4, (uint64_t)n_all * 4};
    };
    if (any_overlap({dspan(g), dspan(e), dspan(u), flat(out_vals, total_k, 4),
                     flat(out_idx, total_k, 4)}))
      return GC_ERR_INVALID_ARG;
  }
  if (n_seg == 0) return GC_OK;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return GC_ERR_HIP;
  char* base = nullptr;
  if (int rc = na_scratch(dev, &base)) return rc;
  gc::DevPlan d{};
  if (na_layout(base, d) > kScratchBytes) return GC_ERR_UNSUPPORTED;
  d.n_seg = n_seg;
  d.flags = (int32_t)(flags | gc::kFlagNoEstimate);
  d.n_tiles = tiles;
  d.n_chunks = chunks;
  d.n_chunk_blocks = gc::chunk_walkers(chunks);
  d.single = 0;
  d.keys = gc::kKeysMagnitude;
  d.n_sample = 0;
  d.sample_tile = nullptr;
  d.gscale = nullptr;
  hipStream_t st = static_cast<hipStream_t>(stream);
  k_noalloc_setup<<<1, 1024, 0, st>>>(d, a);
  hipError_t err = hipGetLastError();
  if (err == hipSuccess)
    err = gc::launch_compress(d, g, e, u, momentum, out_vals, out_idx, gc::Int8Args{}, false,
                              st, nullptr, nullptr);
  return err == hipSuccess ? GC_OK : GC_ERR_HIP;
}

int gc_read_f32(const float* x, int64_t n, uint32_t* sink, void* stream) {
  if (n < 0 || (n && (!x || !sink || !aligned16(x)))) return GC_ERR_INVALID_ARG;
  if (any_overlap({flat(x, n, 4), flat(sink, 64, 4)})) return GC_ERR_INVALID_ARG;
  return gc::launch_read(x, n, sink, static_cast<hipStream_t>(stream)) == hipSuccess
             ? GC_OK
             : GC_ERR_HIP;
}

}  // extern "C"
