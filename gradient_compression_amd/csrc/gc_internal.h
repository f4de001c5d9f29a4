// gc_internal.h -- shared definitions of the HIP kernels and the host plan (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gc {

// Streaming layout: one workgroup of kWaves wave64s per tile of kTile elements.  Wave w owns
// the contiguous range [w*kWaveSpan, (w+1)*kWaveSpan) of its tile; inside it, slot v of lane l
// holds the 4 consecutive elements starting at w*kWaveSpan + v*256 + l*4.  Element order in
// the tile is therefore (w, v, l, c), which is index order: every ordered rank follows it.
// Tile geometry and cache policy of the streaming pass (compile-time configuration).
#ifndef GC_TILE_THREADS
#define GC_TILE_THREADS 1024
#endif
#ifndef GC_TILE_SLOTS
#define GC_TILE_SLOTS 2
#endif
#ifndef GC_NT_LOAD_G        // gradient loads marked non-temporal
#define GC_NT_LOAD_G 1
#endif
#ifndef GC_NT_LOAD_E        // residual (and velocity) loads marked non-temporal
#define GC_NT_LOAD_E 1
#endif
#ifndef GC_NT_STORE_E       // residual (and velocity) stores marked non-temporal
#define GC_NT_STORE_E 1
#endif
// Band of candidates-per-k that the threshold estimate steers toward (one step per call).
#ifndef GC_RHO_LOW
#define GC_RHO_LOW 1.25f
#endif
#ifndef GC_RHO_HIGH
#define GC_RHO_HIGH 2.25f
#endif
#ifndef GC_NT_ZERO_E        // the scattered residual zeroing of kept entries non-temporal
#define GC_NT_ZERO_E 1
#endif
#ifndef GC_SAMPLE_MARGIN    // cold start: capture this many first-key digits below the sample's
#define GC_SAMPLE_MARGIN 2  // estimate of the k-th key (a digit is a factor of 2^(1/8))
#endif
#ifndef GC_BETA_MAX         // largest margin: next threshold <= GC_BETA_MAX * |k-th key|
#define GC_BETA_MAX 0.995f
#endif
// First margin of the threshold estimate (next threshold = beta * |k-th largest|), on a fresh
// plan and after an estimate reset.
constexpr float kInitialBeta = 0.9f;
#ifndef GC_XCD_REMAP        // streaming pass: contiguous tile ranges per XCD
#define GC_XCD_REMAP 0
#endif
constexpr int kThreads = GC_TILE_THREADS;
constexpr int kWaves = kThreads / 64;
constexpr int kSlots = GC_TILE_SLOTS;
constexpr int kWaveSpan = 64 * 4 * kSlots;
constexpr int kTile = kWaves * kWaveSpan;
// Candidate buffers are processed in chunks laid out exactly like tiles.
constexpr int kChunk = kTile;
// Workgroups that serve the exact full-segment path, striding over listed segments.
constexpr int kFullBlocks = 256;
// Workgroups that walk the candidate chunks of a call.  A plan of at most kDirectChunks chunks
// gets one walker per chunk (no list to read first); a larger one kChunkBlocks walkers over the
// chunks that hold candidates, listed per call (a plan has chunks for its full capacity, mostly
// unused).
constexpr int kChunkBlocks = 1024;
constexpr int kDirectChunks = 256;
inline int32_t chunk_walkers(int64_t n_chunks) {
  return (int32_t)(n_chunks <= kDirectChunks ? n_chunks
                                             : (n_chunks < kChunkBlocks ? n_chunks : kChunkBlocks));
}
// Workgroups of the fallback kernels (histograms, re-capture and counts over the tiles of the
// segments whose captured candidates were not complete).
constexpr int kFallbackBlocks = 256;
// Output chunks for the int8 and decompression kernels.
constexpr int kOutChunk = 4096;
constexpr int kHistBins = 2048;
// Segments of at most this many elements are selected whole by one workgroup of the finish
// kernel, their keys held in registers (read from the residual, which holds acc after the
// streaming pass); they capture nothing.
constexpr int64_t kSmallSegment = 16384;
constexpr int kSmallTiles = (int)(kSmallSegment / kTile);
static_assert(kSmallSegment % kTile == 0, "a small segment is a whole number of tiles at most");
// Keys the finish workgroup ranks in its LDS once the range holding the k-th key is this
// small.
constexpr int kListCap = 4096;
// Output chunks whose counts the finish workgroup keeps in LDS at a time.
constexpr int kFinishChunks = 1024;

// Plans whose every segment is small, or has at most kSingleMaxElems elements and either
// 4 k <= kChunk or at most kSingleWholeElems elements, are selected after the pass by one
// workgroup per segment (k_single): its candidates, when complete, selected and emitted in
// index order; otherwise a radix select over the whole segment streamed by that workgroup.
constexpr int64_t kSingleMaxElems = (int64_t)1 << 22;
constexpr int64_t kSingleWholeElems = 65536;
inline bool single_segment_ok(int64_t n, int64_t k) {
  return n <= kSmallSegment ||
         (n <= kSingleMaxElems && (4 * k <= kChunk || n <= kSingleWholeElems));
}

constexpr uint32_t kNoCapture = 0xFFFFFFFFu;        // threshold above every key
// Per-segment path of a call.  kModeCand: the candidates captured at the estimated threshold
// hold the k largest.  kModeRecap: they did not, the segment's first-digit histogram was
// taken and the candidates re-captured at the exact bucket floor.  kModeFull: the bucket is
// larger than the capacity (or forced): radix select over the whole segment.  kModeSmall: a
// small segment, selected whole from its residual by one workgroup.
enum : uint32_t {
  kModeSkip = 0, kModeCand = 1, kModeFull = 2, kModeRecap = 3, kModePending = 4, kModeSmall = 5
};
// Per-segment plan flags.
constexpr uint32_t kSegSmall = 0x1;
// Plan flags seen by the kernels (same values as the public ones).
constexpr int32_t kFlagMomentumMask = 0x1;
constexpr int32_t kFlagForceFull = 0x100;
constexpr int32_t kFlagNoEstimate = 0x200;
constexpr int32_t kFlagChain = 0x400;
// What the select ranks: |acc| (Top-k, threshold) or a per-element Philox key (Random-k).
// Random keys are 31-bit and travel through the candidate buffers as float bit patterns, so
// the select kernels read both kinds through the same magnitude-key view.
enum : int32_t { kKeysMagnitude = 0, kKeysRandom = 1 };
// Which codec a call of the shared select runs for.
enum : int32_t { kCodecTopk = 0, kCodecThreshold = 1, kCodecRandk = 2 };

// Device view of a plan, passed by value to every kernel.
//
// Per-call counters (cand_cnt, recap_cnt, tau_cnt, near_cnt) and the digit histograms are
// zero at the start of every call: the plan starts them at zero and the finish kernel clears
// what a call used once it no longer needs it.  The call's lists (pending, active chunks,
// full path) and the error flag are cleared by the streaming pass's first workgroup.
struct DevPlan {
  int32_t n_seg;
  int32_t flags;
  int64_t n_tiles;
  int64_t n_chunks;
  int32_t n_chunk_blocks;      // chunk_walkers(n_chunks): the chunk walkers of a launch
  int32_t single;              // one workgroup per segment selects after the pass (k_single)
  int32_t codec;               // kCodec* of this call
  // host-built tables
  const int64_t* seg_off;      // [n_seg + 1]
  const int64_t* tile_base;    // [n_seg + 1] first tile of each segment
  const int32_t* tile_seg;     // [n_tiles]
  const int4* tile_desc;       // [n_tiles] {start low 32, start high 32, length, segment}
  const int64_t* chunk_base;   // [n_seg + 1] first candidate chunk of each segment
  const int32_t* chunk_seg;    // [n_chunks]
  const uint32_t* k;           // [n_seg]
  const int64_t* out_off;      // [n_seg + 1]
  const int64_t* cand_base;    // [n_seg] start of the segment's candidate region
  const uint32_t* cand_cap;    // [n_seg] its capacity
  const uint32_t* thr_init;    // [n_seg] threshold of a fresh plan
  const uint32_t* seg_flags;   // [n_seg] kSeg* flags
  // per-segment state
  uint32_t* thr;               // capture threshold of the next call (Random-k: the plan's)
  uint32_t* cand_cnt;          // candidates captured by this call's streaming pass
  uint32_t* recap_cnt;         // candidates re-captured by the fallback
  uint32_t* mode;
  uint32_t* thr_lo;            // re-capture floor of the call
  uint32_t* pfx1;              // full path: prefix after the first digit, and the rank left
  uint32_t* kk1;
  uint32_t* pfx2;              // full path: prefix after the second digit, and the rank left
  uint32_t* kk2;
  uint32_t* kth;               // k-th largest key
  uint32_t* ties;              // entries taken at exactly kth
  uint32_t* sel_cnt;           // candidates the select ran over (emission and statistics)
  uint32_t* hist;              // [n_seg][3][kHistBins]
  uint32_t* full_list;         // [n_seg] segments on the exact full-segment path
  uint32_t* full_count;        // [1]
  uint32_t* pend_list;         // [n_seg] segments whose captured candidates were not complete
  uint32_t* pend_count;        // [1]
  uint32_t* near_cnt;          // [n_seg] candidates in the range that holds the k-th key
  float* beta;                 // [n_seg] threshold margin: next threshold = beta * |kth|
  uint32_t* err;               // [1] internal consistency flag (0 = fine)
  uint32_t* tile_max;          // [n_tiles] largest key of a full-path tile (int8 absmax)
  double* tile_l1;             // [n_tiles] per-tile sum |acc| (sign) or sum acc^2 (QSGD)
  const int64_t* word_off;     // [n_seg + 1] first 32-bit word of each segment's sign bits
  // per-tile state
  uint32_t* run_off;           // [n_tiles] offset of the tile's run in its segment region
  uint32_t* run_cnt;           // [n_tiles]
  uint32_t* run_dst;           // [n_tiles] index-ordered position of the run
  uint32_t* tile_gt;           // [n_tiles] (full-segment path) keys above kth
  uint32_t* tile_eq;           // [n_tiles] keys equal to kth
  uint32_t* tile_eq_base;      // [n_tiles] ties before the tile
  uint32_t* tile_sel_base;     // [n_tiles] kept entries before the tile
  // per-chunk state (candidate path)
  uint32_t* chunk_gt;          // [n_chunks] keys above kth in the chunk
  uint32_t* chunk_max;         // [n_chunks] largest key of the chunk (int8 absmax)
  uint32_t* chunk_eq;          // [n_chunks] keys equal to kth in the chunk
  uint32_t* chunk_eq_base;     // ties before the chunk
  uint32_t* chunk_sel_base;    // kept entries before the chunk
  uint32_t* act_chunk;         // [n_chunks] the chunks that hold candidates this call, any order
  uint32_t* act_count;         // [1] their number
  // candidate buffers, segment s at [cand_base[s], cand_base[s] + cand_cap[s])
  float* cand_val;
  int32_t* cand_idx;
  float* sort_val;             // the same candidates in ascending index order
  int32_t* sort_idx;
  // threshold and Random-k state
  const uint32_t* thr_rand;    // [n_seg] Random-k capture threshold (fixed per plan)
  const float* rk_scale;       // [n_seg] fl32(n / k), Random-k value scale without feedback
  uint32_t* thr_est;           // [n_seg] threshold calls: capture floor estimate (kNoCapture:
                               // none); the capture runs at max(key(tau), floor)
  float* beta_est;             // [n_seg] its margin
  uint32_t* tau_cnt;           // [n_seg] entries with key >= key(|tau|) counted by the capture
  float* seg_norm;             // [n_seg] l2 norms of a clipping call (when the caller wants none)
  const float* gscale;         // [n_seg] caller's gradient scale applied on load, or null
  // per call
  const float* tau;            // threshold call: per-segment thresholds
  int32_t* out_count;          // threshold call: entries kept per segment, or null
  float* scales;               // fused int8: per-segment scales written by the select
  // cold-start sample: about 64 evenly spaced tiles of each large segment
  int64_t n_sample;
  const int32_t* sample_tile;  // [n_sample] tiles whose acc is histogrammed on a cold call
  const int64_t* sample_elems; // [n_seg] elements in the segment's sample (0: not sampled)
  int32_t keys;                // kKeysMagnitude or kKeysRandom
  uint32_t seed_lo, seed_hi, step_lo;   // Random-k key stream
};

struct OutPlan {               // tables of the int8 and decompression kernels
  int32_t n_seg;
  int64_t n_out_chunks;
  const int64_t* seg_off;
  const int64_t* out_off;
  const int32_t* out_chunk_seg;    // [n_out_chunks]
  const int64_t* out_chunk_base;   // [n_seg + 1]
};

// Quantisation fused into the compress call (enabled == 0: plain compress).
struct Int8Args {
  int enabled;
  int8_t* codes;
  float* scales;
  uint32_t seed_lo, seed_hi, step_lo;
};

// The streaming pass of a Top-k (count_tau false) or threshold (true) call (gc_pass.hip):
// acc = e + (u = m u + g | g) written into e (and u), candidates captured per tile.
void launch_ef_capture(const DevPlan& P, const float* g, float* e, float* u, float m,
                       bool count_tau, hipStream_t st);

// Launchers (gc_topk.hip, gc_codecs.hip, gc_scatter.hip).  Each returns the hipError_t of
// its launches.
// cold: the plan has no threshold estimate yet; a sample of tiles sets a first one.
hipError_t launch_compress(const DevPlan& P, const float* g, float* e, float* u, float m,
                           float* out_vals, int32_t* out_idx, const Int8Args& q8, bool cold,
                           hipStream_t st, hipEvent_t ev_begin, hipEvent_t ev_end);
hipError_t launch_threshold(const DevPlan& P, const float* g, float* e, float* u, float m,
                            const float* tau, float* out_vals, int32_t* out_idx,
                            int32_t* out_count, hipStream_t st, hipEvent_t ev_begin,
                            hipEvent_t ev_end);
hipError_t launch_randk(const DevPlan& P, const float* g, float* e, float* u, float m,
                        uint64_t seed, uint64_t step, float* out_vals, int32_t* out_idx,
                        hipStream_t st, hipEvent_t ev_begin, hipEvent_t ev_end);
// factors null: scale g in place where clipped; else write the per-segment factors only.
hipError_t launch_clip(const DevPlan& P, float* g, const float* max_norm, float* norms,
                       float* factors, hipStream_t st);
hipError_t launch_reset(const DevPlan& P, hipStream_t st);
hipError_t launch_sign(const DevPlan& P, const float* g, float* e, float* u, float m,
                       uint32_t* bits, float* scales, hipStream_t st, hipEvent_t ev_begin,
                       hipEvent_t ev_end);
hipError_t launch_qsgd(const DevPlan& P, const float* g, float* e, float* u, float m,
                       int levels, uint64_t seed, uint64_t step, int8_t* codes, float* norms,
                       hipStream_t st, hipEvent_t ev_begin, hipEvent_t ev_end);
hipError_t launch_qsgd_decompress(const DevPlan& P, const int8_t* codes, const float* norms,
                                  int levels, float* dense, int accumulate, hipStream_t st);
hipError_t launch_sign_decompress(const DevPlan& P, const uint32_t* bits, const float* scales,
                                  float* dense, int accumulate, hipStream_t st);
hipError_t launch_quant(const OutPlan& O, const float* vals, const int32_t* idx, float* e,
                        uint64_t seed, uint64_t step, int8_t* codes, float* scales,
                        hipStream_t st);
hipError_t launch_decompress(const OutPlan& O, const float* vals, const int8_t* codes,
                             const float* scales, const int32_t* idx, float* dense,
                             int accumulate, hipStream_t st);
hipError_t launch_fill_zero(float* dense, int64_t a, int64_t b, hipStream_t st);
hipError_t launch_copy(const float* src, float* dst, int64_t n, hipStream_t st);

}  // namespace gc
