/*
 * gc.h -- C ABI of the MI355X (gfx950) error-feedback gradient compressors.
 *
 * The main path is error-feedback Top-k (below).  The same plan also serves threshold and
 * Random-k sparsification, 1-bit sign and QSGD codecs, local gradient clipping, and the
 * receiver-side sum of several workers' payloads; each entry point states its own
 * definition and source.
 *
 * The operation, per segment (one parameter tensor) of a worker's flat fp32 gradient,
 * is the error-feedback Top-k step of "Communication Optimization > Gradient Compression"
 * (Top-K section, the two displayed equations):
 *     acc = g + e_prev          (e_prev: the local residual of everything not yet sent)
 *     g^  = TopK(acc)           (keep the k entries of largest |acc|, zero the rest)
 *     e   = acc - g^            (the dropped mass stays local for the next step)
 * with optional momentum correction first ("Gradient Sparsification" glossary, momentum
 * sections: the velocity is updated with the dense local gradient before sparsification):
 *     u = m*u + g ;  acc = e_prev + u
 * The kept entries travel as an fp32 value plus a 32-bit index each (Top-K section,
 * wire-format paragraph), optionally quantised to int8 with one scale per segment
 * ("Gradient Compression" glossary: Top-k then 8-bit; "Communication Optimization >
 * Gradient Compression": layer-wise scaling, stochastic rounding that keeps E[Q(x)] = x).
 *
 * Exact semantics (the results are unique and bit-exact):
 *   - every fp32 operation is one IEEE binary32 operation, round to nearest even, no fused
 *     multiply-add, denormals kept: u = fl(fl(m*u) + g), acc = fl(e + x);
 *   - |acc| is ordered through the key bits(acc) & 0x7FFFFFFF (so -0 ties +0); among equal
 *     magnitudes the lower index is kept first;
 *   - the kept entries of a segment are written in ascending segment-local index order;
 *   - the residual is +0.0 at a kept position and acc elsewhere.
 *   - NaN inputs are outside the contract.
 *
 * All pointers are device pointers unless marked "host".  Calls are asynchronous on
 * `stream`, a hipStream_t passed as void* (NULL = the default stream).  The signatures take
 * void* so that this header needs no HIP include and callers that only hold an opaque
 * handle (ctypes, torch's stream pointer) pass it unchanged: arguments are checked on the host
 * before anything is launched, and errors of the launched work surface at the caller's
 * next synchronisation.  No call allocates device memory except gc_plan_create.  A plan
 * serves one stream at a time; calls on one plan must not overlap.  The buffers of one call
 * must not share any byte (a dense buffer spans elements [seg_off[0], seg_off[n_seg]), the
 * others their stated length); the host check rejects a violation with GC_ERR_INVALID_ARG.
 * No exception crosses this interface; every function returns a gc_status (0 = success).
 */
#ifndef GC_H
#define GC_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GC_OK = 0,
    GC_ERR_INVALID_ARG = -1,   /* a bad argument; nothing was launched */
    GC_ERR_OOM = -2,           /* device memory for the plan could not be allocated */
    GC_ERR_HIP = -3,           /* the HIP runtime reported an error (no device, launch failure) */
    GC_ERR_UNSUPPORTED = -4    /* a valid request the library does not handle */
} gc_status;

/* Plan flags. */
#define GC_MOMENTUM_MASK 0x1u         /* also zero the velocity u at the kept positions
                                         (momentum factor masking, "Gradient
                                         Sparsification" glossary, DGC section) */
#define GC_DEBUG_FORCE_FALLBACK 0x100u /* every segment takes the exact radix select over
                                          the whole segment (same results, slower; tests) */
#define GC_DEBUG_NO_ESTIMATE 0x200u    /* keep no threshold between calls: every call
                                          re-captures candidates from a histogram of the
                                          whole segment (same results, slower; tests) */
#define GC_DEBUG_CHAIN 0x400u          /* select with the chain of kernels over candidate
                                          chunks even where one workgroup per segment would
                                          do (same results; tests) */

typedef struct gc_plan gc_plan;

/*
 * Host-only (no GPU needed): the k per segment and the output layout a plan with these
 * arguments has, with the checks of gc_plan_create on seg_off, k and ratio.
 *   k_out   : host int64[n_seg] receiving k[s], or NULL.
 *   out_off : host int64[n_seg + 1] receiving the exclusive prefix sum of k, or NULL.
 * Errors: GC_ERR_INVALID_ARG.
 */
int gc_layout(const int64_t* seg_off, int32_t n_seg, const int64_t* k, const double* ratio,
              int64_t* k_out, int64_t* out_off);

/*
 * Build a plan for a segmented buffer and allocate its device workspace on the current
 * device.
 *   seg_off : host int64[n_seg + 1], non-decreasing, seg_off[0] >= 0; segment s covers
 *             elements [seg_off[s], seg_off[s+1]) of g, e and u; each segment < 2^31 elements.
 *   n_seg   : number of segments, >= 0.
 *   k       : host int64[n_seg], 0 <= k[s] <= segment size; or NULL when ratio is given.
 *   ratio   : host double[n_seg] in [0, 1]; k[s] = min(n_s, ceil(n_s * ratio[s])) computed in
 *             exact parts-per-billion (0.1% of 2^20 gives 1049); or NULL when k is given.
 *             Exactly one of k and ratio must be non-NULL.
 *   flags   : any of GC_MOMENTUM_MASK, GC_DEBUG_FORCE_FALLBACK, GC_DEBUG_NO_ESTIMATE,
 *             GC_DEBUG_CHAIN, or 0.
 *   out     : receives the plan.
 * The plan keeps a per-segment threshold estimate between calls; it only decides how much
 * work a call does, never what it returns.  Where every segment is modest (at most 4M
 * elements with 4 k[s] <= 8192, or at most 65536 elements, at the default tile geometry) a
 * call selects with one workgroup per segment after its streaming pass; otherwise with a
 * chain of kernels over the candidate chunks; the results are the same.  Its single device
 * allocation holds about 25 KB
 * per segment (three 2048-bin histograms and per-segment state), about 60 B per 8192-element
 * tile, and 16 B per candidate slot (min(n_s, max(16 k_s, 65536)) slots per segment, none for
 * segments of at most 16384 elements, which are selected whole): about 1.8 GB for a
 * 6.7e9-element, 291-segment gradient at k = 0.1%.
 * Errors: GC_ERR_INVALID_ARG (any check above), GC_ERR_OOM (the workspace does not fit),
 * GC_ERR_UNSUPPORTED (2^31 or more tiles, candidate chunks or int8 output chunks, or more
 * than 4 * (2^32 - 1) candidate slots in all: the kernels' 32-bit grid and slot counts;
 * nothing is allocated), GC_ERR_HIP.
 */
int gc_plan_create(const int64_t* seg_off, int32_t n_seg, const int64_t* k, const double* ratio,
                   uint32_t flags, gc_plan** out);

/* Free the plan and its workspace (synchronises the device first).  NULL is accepted. */
int gc_plan_destroy(gc_plan* plan);

/* Sum of k over the segments: the length of vals, idx and codes. */
int gc_plan_total_k(const gc_plan* plan, int64_t* total_k /* host */);

/* Per-segment k (host int64[n_seg]) and the output offsets: out_off[s] is where segment s's
 * kept entries start, out_off[n_seg] = total k (host int64[n_seg + 1]).  Either may be NULL. */
int gc_plan_layout(const gc_plan* plan, int64_t* k /* host or NULL */,
                   int64_t* out_off /* host or NULL */);

/*
 * The error-feedback Top-k step over every segment.
 *   g        : float[N] fresh gradient, read only; must not overlap e, u or the outputs.
 *   e        : float[N] residual, read and rewritten in place.
 *   u        : float[N] velocity, updated in place (u = fl(fl(momentum*u) + g)), or NULL for
 *              plain error feedback (momentum is then ignored).
 *   out_vals : float[total_k]; out_idx : int32[total_k] segment-local indices; segment s
 *              writes [out_off[s], out_off[s+1]) in ascending index order.
 * N = seg_off[n_seg]; elements outside the segments are not touched.  g, e and u must be
 * 16-byte aligned.
 * Errors: GC_ERR_INVALID_ARG (NULL, misaligned or overlapping buffers), GC_ERR_HIP (launch
 * failure).
 */
int gc_topk_ef_compress(gc_plan* plan, const float* g, float* e, float* u, float momentum,
                        float* out_vals, int32_t* out_idx, void* stream);

/*
 * gc_topk_ef_compress for callers that cannot allocate device memory at any point: code
 * under HIP graph capture, tight serving loops, harnesses that forbid allocation.  It takes
 * the segment table instead of a plan and allocates nothing (no hipMalloc, no hipFree, no
 * host heap): its per-call state lives in a static device array of 24 MiB that the library
 * holds on each device it runs on until the process ends, set up afresh by a small kernel at
 * the start of every call.  The results are bit-identical to gc_topk_ef_compress on a plan
 * made from the same arguments; there is no threshold estimate between calls, so every
 * segment takes the exact re-capture (or full-segment) path, which is slower than a warm plan.
 *   seg_off, n_seg, k, ratio : as for gc_plan_create (host arrays, read during the call).
 *   flags    : GC_MOMENTUM_MASK or 0.
 *   g, e, u, momentum, out_vals, out_idx, stream : as for gc_topk_ef_compress (out_off is
 *              the exclusive prefix sum of k).
 * Limits: n_seg <= GC_NOALLOC_MAX_SEGMENTS, seg_off[n_seg] - seg_off[0] <=
 * GC_NOALLOC_MAX_ELEMENTS, and the candidate capacity, sum over segments of
 * min(n_s, max(4 k_s, 65536)), at most GC_NOALLOC_MAX_CANDIDATES; beyond them the call
 * returns GC_ERR_UNSUPPORTED and launches nothing.  Every call on a device uses that device's
 * one array, which keeps the last call's contents: calls that overlap on one device (other
 * streams, other threads) race and must be serialised by the caller.
 * Errors: GC_ERR_INVALID_ARG, GC_ERR_UNSUPPORTED, GC_ERR_HIP.
 */
#define GC_NOALLOC_MAX_SEGMENTS 64
#define GC_NOALLOC_MAX_ELEMENTS (1ll << 22)
#define GC_NOALLOC_MAX_CANDIDATES (1ll << 20)
int gc_topk_ef_compress_noalloc(const int64_t* seg_off /* host */, int32_t n_seg,
                                const int64_t* k /* host or NULL */,
                                const double* ratio /* host or NULL */, uint32_t flags,
                                const float* g, float* e, float* u, float momentum,
                                float* out_vals, int32_t* out_idx, void* stream);

/*
 * Quantise the kept values to int8, one scale per segment, with stochastic rounding:
 *   scale_s = fl(absmax_s / 127) over the segment's kept values (0 when all are 0);
 *   a = min(fl(|v| / scale_s), 127); q = floor(a) + [u24 < (a - floor(a)) * 2^24];
 *   code = sign(v) * q  (0 when scale_s is 0)
 * where u24 is the top 24 bits of word 0 of Philox4x32-10 (Salmon et al., SC'11) keyed by
 * (seed low 32 bits, seed high 32 bits) at counter (global index low 32, global index high
 * 32, step low 32, 0x51), global index = seg_off[s] + idx.
 *   vals, idx : as written by gc_topk_ef_compress (total_k entries).
 *   e         : float[N] residual or NULL; when given, the quantisation error is fed back:
 *               e[seg_off[s] + idx] = fl(v - fl(code * scale_s)).
 *   out_codes : int8[total_k]; out_scales : float[n_seg].
 * Errors: GC_ERR_INVALID_ARG, GC_ERR_HIP.
 */
int gc_quant_int8(gc_plan* plan, const float* vals, const int32_t* idx, float* e, uint64_t seed,
                  uint64_t step, int8_t* out_codes, float* out_scales, void* stream);

/*
 * The compress step and the int8 stage in one call: the same results, bit for bit, as
 * gc_topk_ef_compress followed by gc_quant_int8 with the residual e (the quantisation error
 * is fed back into e), with one emission pass instead of two.  The per-segment absmax is
 * the segment's largest |acc|, which is always kept.
 *   out_vals  : float[total_k] kept fp32 values, or NULL when only the codes are wanted.
 *   out_idx   : int32[total_k]; out_codes : int8[total_k]; out_scales : float[n_seg].
 *   other arguments as for gc_topk_ef_compress and gc_quant_int8.
 * Errors: GC_ERR_INVALID_ARG, GC_ERR_HIP.
 */
int gc_topk_ef_compress_int8(gc_plan* plan, const float* g, float* e, float* u, float momentum,
                             uint64_t seed, uint64_t step, float* out_vals, int32_t* out_idx,
                             int8_t* out_codes, float* out_scales, void* stream);

/*
 * The receiver's step: rebuild the sparse update from a payload of (value, index) pairs
 * ("Communication Optimization > Gradient Compression", Top-K section, wire-format
 * paragraph: each kept entry travels as its value and its position; "Gradient Compression"
 * memory-compression glossary, systems section: the values and indices that workers exchange
 * are what the receiver adds up; an int8 payload is dequantised with the per-segment scale
 * that travels alongside it, layer-wise scaling paragraph).
 * Scatter kept entries back into a dense float[N] buffer: dense[seg_off[s] + idx] = v, with
 * v = vals[j] when vals is given, else fl(codes[j] * scales[s]).  accumulate = 0 first sets
 * dense to +0 over [seg_off[0], N); accumulate != 0 adds v instead of storing it.  Entries
 * with index -1 (the padding of a threshold call) are skipped.
 *   vals  : float[total_k] in the plan's layout (out_off), or NULL when codes are given.
 *   codes : int8[total_k], or NULL; scales : float[n_seg] (with codes).
 *   idx   : int32[total_k] segment-local indices; dense : float[N], owned by the caller.
 * Exactly one of vals and codes must be non-NULL (scales with codes).
 * Errors: GC_ERR_INVALID_ARG (nothing launched), GC_ERR_HIP.
 */
int gc_decompress(const gc_plan* plan, const float* vals, const int8_t* codes,
                  const float* scales, const int32_t* idx, float* dense, int accumulate,
                  void* stream);

/*
 * 1-bit sign compression with error feedback ("Communication Optimization > Gradient
 * Compression", 1-bit SGD section: Q(g) = sign(g) * ||g||_1 / d with the scalar computed
 * per layer; its QSGD paragraph: 1-bit needs error feedback, as top-K does).  Per segment
 * of n elements, after the same momentum and EF add as gc_topk_ef_compress:
 *   scale = fl32(S / n), S = sum |acc| accumulated in double (summation order unspecified:
 *           the scale may differ from the exactly rounded value by 1 ulp);
 *   sign  = -1 where acc < 0, else +1 (zeros of either sign send +1);
 *   bit i of the segment (word i/32, bit i%32, least significant first) = 1 for sign -1;
 *   e = fl(acc - sign * scale).
 * The plan's k is not used (a plan with k = 0 serves).  out_bits: uint32[word_off[n_seg]]
 * with the segment offsets of gc_plan_sign_layout; out_scales: float[n_seg].
 * g, e and u must be 16-byte aligned.  Errors: GC_ERR_INVALID_ARG, GC_ERR_HIP.
 */
int gc_sign_ef_compress(gc_plan* plan, const float* g, float* e, float* u, float momentum,
                        uint32_t* out_bits, float* out_scales, void* stream);

/* First 32-bit word of each segment's sign bits, word_off[s+1] - word_off[s] = ceil(n_s/32)
 * (host int64[n_seg + 1]). */
int gc_plan_sign_layout(const gc_plan* plan, int64_t* word_off);

/* dense[seg_off[s] + i] = sign_i * scale_s (or += with accumulate) over every segment. */
int gc_sign_decompress(const gc_plan* plan, const uint32_t* bits, const float* scales,
                       float* dense, int accumulate, void* stream);

/*
 * QSGD with `levels` = s levels ("Communication Optimization > Gradient Compression", QSGD
 * paragraph: Q_s(g) = ||g|| sgn(g) xi(g, s) / s with xi the stochastic rounding of
 * |g| / (||g|| / s), so that E[Q_s(g)] = g; the printed formula lacks the 1/s, restored
 * here; s = 2^b - 1 gives b-bit levels), one l2 norm per segment.  Per segment:
 *   acc = e + x with error feedback (e given; genomic-FL glossary: quantisation combined
 *         with error feedback), else acc = x; x = g, or u = fl(fl(m*u) + g) with momentum;
 *   norm = fl32(sqrt(S)), S = sum acc^2 in double (order unspecified: 1 ulp);
 *   step = fl32(norm / s); a = min(fl32(|acc| / step), s);
 *   code = sgn(acc) * (floor(a) + [u24 < frac(a) * 2^24]), u24 the top 24 bits of word
 *          (global index % 4) of the Philox4x32-10 block keyed (seed lo, seed hi) at counter
 *          (global index / 4 lo, hi, step lo, 0x52); code = 0 when step is 0;
 *   with e: e = fl(acc - fl(code * step)).
 *   levels   : s in [1, 127] (codes fit int8 with the sign).
 *   e        : float[N] residual (error feedback) or NULL for plain QSGD.
 *   out_codes: int8[N], element i of the buffer at byte i (4-byte aligned).
 *   out_norms: float[n_seg].
 * g, e and u must be 16-byte aligned.  Errors: GC_ERR_INVALID_ARG, GC_ERR_HIP.
 */
int gc_qsgd_compress(gc_plan* plan, const float* g, float* e, float* u, float momentum,
                     int32_t levels, uint64_t seed, uint64_t step, int8_t* out_codes,
                     float* out_norms, void* stream);

/* dense[i] = fl(code_i * fl(norm_s / levels)) (or += with accumulate) over every segment. */
int gc_qsgd_decompress(const gc_plan* plan, const int8_t* codes, const float* norms,
                       int32_t levels, float* dense, int accumulate, void* stream);

/*
 * Threshold sparsification with error feedback (genomic-FL glossary, sparsification section:
 * an entry is sent only if its magnitude reaches a threshold, which may be fixed or may
 * adapt; "Gradient Sparsification" glossary, mechanism section: the threshold may change
 * per layer and step).
 * Per segment, after the same momentum and EF add as gc_topk_ef_compress, the entries with
 * |acc| >= |tau_s| are kept, at most k_s of them (the plan's k is the cap): when more reach
 * the threshold, the k_s largest by (|acc| descending, index ascending).
 *   tau       : device float[n_seg], one threshold per segment (|tau| is used; not NaN).
 *   out_vals, out_idx : the plan's layout; segment s writes its c_s kept entries in
 *               ascending index order at out_off[s], and the slots [c_s, k_s) get value +0
 *               and index -1 (gc_decompress skips them).
 *   out_count : device int32[n_seg] receiving c_s, or NULL.
 *   e         : +0 at the kept positions, acc elsewhere; u zeroed there with
 *               GC_MOMENTUM_MASK.
 * Candidates are captured at max(|tau_s|, a floor estimated from the last threshold calls'
 * k-th kept magnitude), so that a threshold that many entries reach stays on the fast path;
 * the result does not depend on the floor.  The Top-k threshold estimate of the plan is not
 * touched.  Same alignment and aliasing rules as gc_topk_ef_compress.
 * Errors: GC_ERR_INVALID_ARG, GC_ERR_HIP.
 */
int gc_threshold_ef_compress(gc_plan* plan, const float* g, float* e, float* u, float momentum,
                             const float* tau, float* out_vals, int32_t* out_idx,
                             int32_t* out_count, void* stream);

/*
 * Random-k sparsification ("Gradient Compression", memory-compression glossary, Random-k
 * section: a random mask per iteration, no sort of the gradient, unbiased; genomic-FL
 * glossary, sparsification section: random sparsification).
 * Per segment exactly k_s positions, the k_s largest of a 31-bit key per element -- word
 * (gi % 4) of the Philox4x32-10 block keyed (seed lo, seed hi) at counter (gi / 4 lo, gi / 4
 * hi, step lo, 0x53), shifted right by one; gi the global element index; equal keys go to
 * the lower index.  Ranking by independent uniform keys draws a uniformly random k-subset;
 * the mask depends on (seed, step, gi) only, so every worker can rebuild it.
 *   x = g, or with u the momentum-corrected u = fl(fl(m*u) + g) (written back);
 *   e given (error feedback): acc = fl(e + x), out_vals = acc at the mask, e = +0 there and
 *         acc elsewhere;
 *   e NULL: out_vals = fl(x * fl32(n_s / k_s)) at the mask (n_s / k_s formed in double),
 *         whose expectation is x; nothing else is read for the plain case (g is gathered at
 *         the mask only).
 *   out_vals, out_idx : the plan's layout, ascending index per segment.
 *   u zeroed at the mask with GC_MOMENTUM_MASK.
 * g, e and u must be 16-byte aligned.  Errors: GC_ERR_INVALID_ARG, GC_ERR_HIP.
 */
int gc_randk_compress(gc_plan* plan, const float* g, float* e, float* u, float momentum,
                      uint64_t seed, uint64_t step, float* out_vals, int32_t* out_idx,
                      void* stream);

/*
 * Local gradient clipping ("Gradient Compression", genomic-FL glossary, DGC section: the
 * gradient magnitude is normalised before compression; memory-compression glossary,
 * quantization section: clipping before quantisation controls the range), the l2 reading,
 * per segment s, in place on g before a compress call:
 *   norm_s = fl32(sqrt(S)), S = sum g_i^2 in double (order unspecified: within 1 ulp);
 *   when norm_s > max_norm[s]: g_i = fl(g_i * fl32(max_norm[s] / norm_s)); else g untouched.
 *   max_norm  : device float[n_seg], >= 0 (0 clears every non-zero segment).
 *   norms_out : device float[n_seg] receiving norm_s before clipping, or NULL.
 * g must be 16-byte aligned; inputs with Inf or NaN are outside the contract.
 * Errors: GC_ERR_INVALID_ARG, GC_ERR_HIP.
 */
int gc_clip_by_norm(gc_plan* plan, float* g, const float* max_norm, float* norms_out,
                    void* stream);

/*
 * Clipping folded into the compress calls.  gc_clip_factors runs only the norm pass of
 * gc_clip_by_norm and writes, per segment, f_s = fl32(max_norm[s] / norm_s) where
 * norm_s > max_norm[s], else 1 (factors_out: device float[n_seg]; g is not modified).
 * gc_plan_set_gradient_scale(plan, factors) makes every later compress call of the plan
 * (Top-k, int8, threshold, Random-k, sign, QSGD) use x = fl(g_i * f_s) wherever it reads g,
 * which is bit-identical to gc_clip_by_norm followed by that call, without its 8 B/element
 * scaling pass; NULL switches it off.  The factors array must stay valid while it is set.
 * Errors: GC_ERR_INVALID_ARG, GC_ERR_HIP.
 */
int gc_clip_factors(gc_plan* plan, const float* g, const float* max_norm, float* norms_out,
                    float* factors_out, void* stream);
int gc_plan_set_gradient_scale(gc_plan* plan, const float* factors);

/*
 * Receiver side of the data-parallel exchange ("Gradient Compression", memory-compression
 * glossary, systems section: sparse gradients are exchanged by all-gather of values and
 * indices; "Communication Optimization > Gradient Compression", subtlety paragraph: the
 * workers' supports differ, so the union is denser than one payload).  The payloads of
 * n_workers workers, gathered back to back in worker order, are added into dense one worker
 * after the other:
 *   dense = 0 unless accumulate; then for w = 0, 1, ..., n_workers - 1 and every entry j of
 *   worker w: dense[seg_off[s] + idx] = fl(dense[...] + value), value = vals[j] or
 *   fl(codes[j] * scales[w * n_seg + s]); entries with an index outside the segment (the -1
 *   padding of threshold payloads) are skipped.
 * The fp32 additions happen in worker order, so every receiver forms the same sum.
 *   vals / codes, idx : device arrays of n_workers * total_k entries, worker w's payload
 *                       (the plan's layout) at w * total_k; exactly one of vals and codes.
 *   scales            : with codes, device float[n_workers * n_seg].
 *   dense             : device float[N].
 * Errors: GC_ERR_INVALID_ARG, GC_ERR_HIP.
 */
int gc_decompress_gathered(const gc_plan* plan, int32_t n_workers, const float* vals,
                           const int8_t* codes, const float* scales, const int32_t* idx,
                           float* dense, int accumulate, void* stream);

/* Forget the threshold estimates (of Top-k calls and the capture floor of threshold calls):
 * the next call runs as on a fresh plan. */
int gc_plan_reset_estimate(gc_plan* plan, void* stream);

/*
 * Diagnostics of the last compress call (synchronises `stream`).  Host arrays of n_seg, any
 * may be NULL: mode[s] (0 = k is 0; 1 = selected among the candidates captured at the
 * estimated threshold; 2 = exact radix select over the whole segment; 3 = candidates
 * re-captured after a histogram of the whole segment; 5 = a segment of at most 16384
 * elements, selected whole by one workgroup), candidates[s] (entries the select ran over:
 * those captured in modes 1 and 3, else 0), kth_key[s] (the k-th largest key
 * bits(acc) & 0x7FFFFFFF), ties_taken[s] (entries kept at exactly that key).  Returns
 * GC_ERR_HIP when the call's kernels raised their internal consistency flag.
 */
int gc_plan_last_stats(gc_plan* plan, uint32_t* mode, uint32_t* candidates, uint32_t* kth_key,
                       uint32_t* ties_taken, void* stream);

/*
 * Timing of the streaming error-feedback pass: when enabled, every compress call records a
 * HIP event pair around that kernel on its stream; gc_plan_timing returns the summed time
 * in milliseconds and the number of launches since the last query (synchronising on the
 * events) and resets both.
 */
int gc_plan_set_timing(gc_plan* plan, int enable);
int gc_plan_timing(gc_plan* plan, double* ms /* host */, int64_t* launches /* host */);

/* Reference streaming kernel for bandwidth calibration: dst[i] = src[i] for n floats with
 * 16-byte loads and stores (n a multiple of 4, both pointers 16-byte aligned). */
int gc_copy_f32(const float* src, float* dst, int64_t n, void* stream);

/* Reference streaming kernel for the error-feedback pass's memory pattern: y[i] = fl(y[i] +
 * x[i]) for n floats (two reads, one write per element) with the pass's tile layout and
 * non-temporal 16-byte loads and stores, and none of its selection work (a reference stream,
 * not a ceiling: the pass streams faster than this bare kernel).  Both pointers
 * 16-byte aligned; x and y must not overlap.  Errors: GC_ERR_INVALID_ARG, GC_ERR_HIP. */
int gc_add_f32(const float* x, float* y, int64_t n, void* stream);

/* Reference pure read stream: reads n floats at x (16-byte aligned) with the pass's tile
 * layout and non-temporal 16-byte loads, and writes nothing (sink, 64 uint32 of device
 * memory, is written only in a case that does not arise for real data).
 * Errors: GC_ERR_INVALID_ARG, GC_ERR_HIP. */
int gc_read_f32(const float* x, int64_t n, uint32_t* sink, void* stream);

/* Static text for a status code. */
const char* gc_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* GC_H */
