/*
 * oracle.c -- plain, slow CPU oracle of error-feedback Top-k gradient compression.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's CPU-baseline
 * leg may load this library.  It shares no code, header, table or constant with the HIP
 * library it checks; it is written from the pages' definitions, not for speed.
 *
 * Compile with -O2 -ffp-contract=off and never -ffast-math: every fp32 operation below is
 * one IEEE-754 binary32 operation with round-to-nearest-even and denormals kept.
 *
 * What it computes, per segment (one parameter tensor), following
 * "Communication Optimization > Gradient Compression" (Top-K section, the two displayed
 * equations  g^_t = TopK(g_t + e_{t-1})  and  e_t = (g_t + e_{t-1}) - g^_t):
 *   1. optional momentum correction, the velocity updated with the dense local gradient
 *      before sparsification ("Gradient Sparsification" glossary, momentum-correction
 *      section): u = fl(fl(m*u) + g), and the vector compressed is x = u; otherwise x = g.
 *   2. acc = fl(e + x).
 *   3. TopK: a FULL SORT of the positions by (|acc| descending, position ascending); the
 *      first k are selected.  |acc| is compared through the 31-bit key bits(acc) & 0x7FFFFFFF,
 *      whose unsigned order is the order of |acc| (so -0 and +0 tie).  Equal magnitudes go
 *      to the lower position, which makes the selected set unique.
 *   4. The selected (value, segment-local index) pairs are emitted in ascending index
 *      order: an fp32 value plus a 32-bit index per entry (Top-K section, wire format).
 *   5. Residual: e = acc - g^, i.e. +0 at the selected positions and acc elsewhere.
 *      With the momentum-mask option the velocity is also zeroed there ("Gradient
 *      Sparsification" glossary, DGC section: the same mask applied to the momentum buffer).
 *
 * Optional 8-bit stage ("Gradient Compression" glossary: Top-k then 8-bit quantisation of
 * the kept values; genomic-FL glossary, quantization section: FP32 -> INT8 with stochastic
 * rounding; "Communication Optimization > Gradient Compression", QSGD and layer-wise
 * scaling paragraphs): per segment scale = fl(absmax/127) over the kept values,
 * a = min(fl(|v|/scale), 127), q = floor(a) + [u24 < frac(a)*2^24], code = sign(v)*q, and
 * the quantisation error is fed back: e = fl(acc - fl(code*scale)).  u24 is the top 24
 * bits of word 0 of Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11) with key (seed lo,
 * seed hi) and counter (global index lo, global index hi, step lo, 0x51).
 *
 * 1-bit sign compression with error feedback ("Communication Optimization > Gradient
 * Compression", 1-bit SGD section): per segment scale = fl32(sum |acc| / n) with the sum
 * in double, one sign bit per element, residual e = fl(acc - sign * scale).
 *
 * Threshold sparsification with error feedback: the entries with |acc| >= tau, at most k of
 * them (the largest), as above otherwise.
 *
 * Random-k ("Gradient Compression", memory-compression glossary, Random-k section; genomic-FL
 * glossary, sparsification section: random sparsification): exactly k positions per segment, a uniformly random subset drawn anew each
 * step -- the k largest of a Philox4x32-10 key per element (counter tag 0x53).  With error
 * feedback the values go unscaled and the residual is kept; without it they are scaled by
 * n/k so that their expectation is acc.
 *
 * Local gradient clipping (genomic-FL glossary, DGC section: the gradient magnitude is
 * normalised before compression; memory-compression glossary, quantization section: clipping
 * before quantisation controls the range): per segment, the l2 norm is brought down to a
 * given bound when it exceeds it.
 *
 * QSGD with s levels (same page, QSGD paragraph, with its missing 1/s restored): one l2
 * norm per segment, stochastic levels drawn from Philox4x32-10 (one block per four
 * consecutive elements, counter tag 0x52), error feedback of the quantisation error optional.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- small helpers */

static uint32_t bits_of(float x) { uint32_t u; memcpy(&u, &x, sizeof u); return u; }

/* Magnitude key: unsigned order of (bits & 0x7FFFFFFF) is the order of |x| for non-NaN x. */
static uint32_t magnitude_key(float x) { return bits_of(x) & 0x7FFFFFFFu; }

/* ------------------------------------------------------------------- k from ratio */

/* k = min(n, ceil(n * ratio)), with ratio taken in exact integer parts per billion so
 * that 0.1% of 2^20 is 1049 and 1% of 6400 is exactly 64.  Returns -1 for a ratio outside
 * [0, 1] and 0 for n <= 0. */
int64_t orc_k_from_ratio(int64_t n, double ratio)
{
    if (!(ratio >= 0.0 && ratio <= 1.0)) return -1;
    if (n <= 0) return 0;
    int64_t ppb = llround(ratio * 1e9);
    __int128 num = (__int128)n * ppb + 999999999;
    int64_t k = (int64_t)(num / 1000000000);
    return k > n ? n : k;
}

/* ------------------------------------------------------------------------- TopK */

typedef struct { uint32_t key; uint32_t pos; } rank_rec;

/* Order of the full sort: key descending, then position ascending. */
static int by_rank(const void* pa, const void* pb)
{
    const rank_rec* a = (const rank_rec*)pa;
    const rank_rec* b = (const rank_rec*)pb;
    if (a->key != b->key) return a->key > b->key ? -1 : 1;
    if (a->pos != b->pos) return a->pos < b->pos ? -1 : 1;
    return 0;
}

static int by_pos(const void* pa, const void* pb)
{
    uint32_t a = *(const uint32_t*)pa, b = *(const uint32_t*)pb;
    return a < b ? -1 : (a > b ? 1 : 0);
}

/*
 * One segment of n elements (n < 2^31), k in [0, n].
 *   g    : fresh gradient, read only
 *   e    : residual, updated in place (acc is formed from it, then the residual written)
 *   u    : velocity or NULL; updated in place when given
 *   m    : momentum factor (used only with u)
 *   mask_u : nonzero -> zero u at the selected positions
 *   vals, idx : k outputs, ascending idx
 * Returns 0, or -1 on a bad argument or allocation failure.
 */
int orc_topk_ef_segment(int64_t n, int64_t k, const float* g, float* e, float* u, float m,
                        int mask_u, float* vals, int32_t* idx)
{
    if (n < 0 || n > 0x7FFFFFFF || k < 0 || k > n) return -1;
    if (n == 0) return 0;

    /* steps 1-2: momentum (optional) and the error-feedback add; acc lives in e */
    for (int64_t i = 0; i < n; ++i) {
        float x = g[i];
        if (u) {
            float mu = m * u[i];
            u[i] = mu + x;
            x = u[i];
        }
        e[i] = e[i] + x;
    }

    /* step 3: full sort by (key desc, position asc) */
    rank_rec* rec = (rank_rec*)malloc((size_t)n * sizeof *rec);
    uint32_t* sel = (uint32_t*)malloc((size_t)(k > 0 ? k : 1) * sizeof *sel);
    if (!rec || !sel) { free(rec); free(sel); return -1; }
    for (int64_t i = 0; i < n; ++i) {
        rec[i].key = magnitude_key(e[i]);
        rec[i].pos = (uint32_t)i;
    }
    qsort(rec, (size_t)n, sizeof *rec, by_rank);

    /* step 4: the first k positions, in ascending order */
    for (int64_t j = 0; j < k; ++j) sel[j] = rec[j].pos;
    free(rec);
    qsort(sel, (size_t)k, sizeof *sel, by_pos);
    for (int64_t j = 0; j < k; ++j) {
        vals[j] = e[sel[j]];
        idx[j] = (int32_t)sel[j];
    }

    /* step 5: residual = acc - g^ : +0 where sent, acc elsewhere */
    for (int64_t j = 0; j < k; ++j) {
        e[sel[j]] = 0.0f;
        if (u && mask_u) u[sel[j]] = 0.0f;
    }
    free(sel);
    return 0;
}

/*
 * Threshold sparsification with error feedback (genomic-FL glossary, sparsification section:
 * an entry is sent only if its magnitude reaches a threshold, which may be fixed or may
 * adapt; "Gradient Sparsification" glossary, mechanism section: a dynamic threshold per
 * layer).  One segment:
 * after the same momentum and EF add, the entries with |acc| >= |tau| are sent, at most
 * k_cap of them -- the k_cap largest by (|acc| descending, position ascending) when more
 * reach the threshold.  Writes *count (the number sent, <= k_cap) and that many outputs in
 * ascending index order; the residual is +0 where sent and acc elsewhere.
 */
int orc_threshold_ef_segment(int64_t n, int64_t k_cap, float tau, const float* g, float* e,
                             float* u, float m, int mask_u, float* vals, int32_t* idx,
                             int64_t* count)
{
    if (n < 0 || n > 0x7FFFFFFF || k_cap < 0 || k_cap > n) return -1;
    /* acc first (as orc_topk_ef_segment would), then count the entries at the threshold */
    float* acc_copy = (float*)malloc((size_t)(n > 0 ? n : 1) * sizeof(float));
    float* u_copy = u ? (float*)malloc((size_t)(n > 0 ? n : 1) * sizeof(float)) : NULL;
    if (!acc_copy || (u && !u_copy)) { free(acc_copy); free(u_copy); return -1; }
    int64_t c = 0;
    for (int64_t i = 0; i < n; ++i) {
        float x = g[i];
        if (u) {
            float mu = m * u[i];
            u_copy[i] = mu + x;
            x = u_copy[i];
        }
        acc_copy[i] = e[i] + x;
        if (magnitude_key(acc_copy[i]) >= magnitude_key(tau)) ++c;
    }
    free(acc_copy);
    free(u_copy);
    int64_t k = c < k_cap ? c : k_cap;
    *count = k;
    /* the k largest entries: all of them reach the threshold */
    return orc_topk_ef_segment(n, k, g, e, u, m, mask_u, vals, idx);
}

/* Whole segmented buffer: segments [seg_off[s], seg_off[s+1]), k[s] entries each, output
 * grouped by segment in segment order.  Returns 0 or -1. */
int orc_topk_ef(int32_t n_seg, const int64_t* seg_off, const int64_t* k, const float* g,
                float* e, float* u, float m, int mask_u, float* vals, int32_t* idx)
{
    int64_t out = 0;
    for (int32_t s = 0; s < n_seg; ++s) {
        int64_t o = seg_off[s], n = seg_off[s + 1] - o;
        int rc = orc_topk_ef_segment(n, k[s], g + o, e + o, u ? u + o : NULL, m, mask_u,
                                     vals + out, idx + out);
        if (rc) return rc;
        out += k[s];
    }
    return 0;
}

/* ---------------------------------------------------------------- Philox4x32-10 */

/* Philox4x32 with 10 rounds, from its definition in Salmon et al. (SC'11): each round
 * multiplies words 0 and 2 by two fixed odd constants, taking the 64-bit products apart
 * into high and low halves, and mixes the high halves with words 1 and 3 and the round
 * key; the key advances by two Weyl constants (golden ratio and sqrt(3) - 1) per round. */
void orc_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4])
{
    const uint32_t mult0 = 0xD2511F53u, mult1 = 0xCD9E8D57u;
    const uint32_t weyl0 = 0x9E3779B9u, weyl1 = 0xBB67AE85u;
    uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
    uint32_t k0 = key_in[0], k1 = key_in[1];
    for (int round = 0; round < 10; ++round) {
        uint64_t p0 = (uint64_t)mult0 * c0;
        uint64_t p1 = (uint64_t)mult1 * c2;
        uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        uint32_t n0 = hi1 ^ c1 ^ k0;
        uint32_t n1 = lo1;
        uint32_t n2 = hi0 ^ c3 ^ k1;
        uint32_t n3 = lo0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
        k0 += weyl0;
        k1 += weyl1;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* Top 24 bits of the stochastic-rounding draw of the element at global index gidx. */
static uint32_t sr_draw24(uint64_t seed, uint64_t step, int64_t gidx)
{
    uint32_t ctr[4] = {(uint32_t)(uint64_t)gidx, (uint32_t)((uint64_t)gidx >> 32),
                       (uint32_t)step, 0x51u};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t r[4];
    orc_philox4x32_10(ctr, key, r);
    return r[0] >> 8;
}

/* ------------------------------------------------------------------ int8 stage */

/*
 * One segment's kept values: kk entries (vals, segment-local idx), segment starting at
 * global index seg_base.  Writes codes[kk] and *scale_out; if e_seg is not NULL (the
 * segment's residual) writes the quantisation error back at the kept positions.
 */
void orc_quant_int8_segment(int64_t kk, const float* vals, const int32_t* idx, int64_t seg_base,
                            float* e_seg, uint64_t seed, uint64_t step, int8_t* codes,
                            float* scale_out)
{
    float absmax = 0.0f;
    for (int64_t j = 0; j < kk; ++j) {
        float a = fabsf(vals[j]);
        if (a > absmax) absmax = a;
    }
    float scale = absmax / 127.0f;
    *scale_out = scale;
    for (int64_t j = 0; j < kk; ++j) {
        float v = vals[j];
        int q = 0;
        if (scale != 0.0f) {
            float a = fabsf(v) / scale;
            if (a > 127.0f) a = 127.0f;
            float f = floorf(a);
            float frac = a - f;
            uint32_t u24 = sr_draw24(seed, step, seg_base + idx[j]);
            q = (int)f + (((float)u24 < frac * 16777216.0f) ? 1 : 0);
        }
        int code = signbit(v) ? -q : q;
        codes[j] = (int8_t)code;
        if (e_seg) {
            float deq = (float)code * scale;
            e_seg[idx[j]] = v - deq;
        }
    }
}

/* Whole buffer: kept values grouped by segment as produced by orc_topk_ef. */
void orc_quant_int8(int32_t n_seg, const int64_t* seg_off, const int64_t* k, const float* vals,
                    const int32_t* idx, float* e, uint64_t seed, uint64_t step, int8_t* codes,
                    float* scales)
{
    int64_t out = 0;
    for (int32_t s = 0; s < n_seg; ++s) {
        orc_quant_int8_segment(k[s], vals + out, idx + out, seg_off[s],
                               e ? e + seg_off[s] : NULL, seed, step, codes + out, &scales[s]);
        out += k[s];
    }
}

/* ------------------------------------------------------------------ decompress */

/* dense[seg_off[s] + idx] = value (or += with accumulate), value = vals[j] when vals is
 * given, else fl(codes[j] * scales[s]).  Without accumulate, dense is zero-filled first.
 * Entries whose index is outside the segment (the -1 padding of a threshold payload) carry
 * nothing and are skipped. */
void orc_decompress(int32_t n_seg, const int64_t* seg_off, const int64_t* k, const float* vals,
                    const int8_t* codes, const float* scales, const int32_t* idx, float* dense,
                    int accumulate)
{
    if (!accumulate)
        for (int64_t i = 0; i < seg_off[n_seg]; ++i) dense[i] = 0.0f;
    int64_t out = 0;
    for (int32_t s = 0; s < n_seg; ++s) {
        for (int64_t j = 0; j < k[s]; ++j) {
            int32_t i = idx[out + j];
            if (i < 0 || i >= seg_off[s + 1] - seg_off[s]) continue;
            float v = vals ? vals[out + j] : (float)codes[out + j] * scales[s];
            float* d = &dense[seg_off[s] + i];
            *d = accumulate ? *d + v : v;
        }
        out += k[s];
    }
}

/* Receiver side of the data-parallel exchange (memory-compression glossary, systems section:
 * sparse gradients travel by all-gather of values and indices): the payloads of n_workers
 * workers, back to back in worker order (worker w's entries from w * K, K = sum of k; codes
 * likewise; scales from w * n_seg), added into dense one worker after the other: dense = 0
 * unless accumulate, then dense[pos] = fl(dense[pos] + value) for worker 0, 1, ...  The fp32
 * additions happen in worker order, so every receiver forms the same sum. */
void orc_decompress_gathered(int32_t n_seg, const int64_t* seg_off, const int64_t* k,
                             int32_t n_workers, const float* vals, const int8_t* codes,
                             const float* scales, const int32_t* idx, float* dense,
                             int accumulate)
{
    int64_t kk = 0;
    for (int32_t s = 0; s < n_seg; ++s) kk += k[s];
    if (!accumulate)
        for (int64_t i = 0; i < seg_off[n_seg]; ++i) dense[i] = 0.0f;
    for (int32_t w = 0; w < n_workers; ++w)
        orc_decompress(n_seg, seg_off, k, vals ? vals + (int64_t)w * kk : NULL,
                       codes ? codes + (int64_t)w * kk : NULL,
                       scales ? scales + (int64_t)w * n_seg : NULL, idx + (int64_t)w * kk,
                       dense, 1);
}

/* ---------------------------------------------------- 1-bit sign with error feedback */

/*
 * One segment of n elements.  "Communication Optimization > Gradient Compression", 1-bit
 * SGD section: Q(g) = sign(g) * ||g||_1 / d, the scalar taken per layer; its QSGD paragraph:
 * 1-bit quantisation needs error feedback like top-K.  With the residual e:
 *   acc = e + x (x = g, or u = m*u + g with momentum);
 *   scale = fl32(S / n), S = sum |acc_i| accumulated in double in index order;
 *   sign_i = -1 where acc_i < 0, +1 otherwise (so -0 and +0 both send +1);
 *   bit i of the segment's bit array (word i/32, bit i%32) is 1 where sign_i = -1;
 *   e_i = fl(acc_i - sign_i * scale).
 * bits: ceil(n/32) words, cleared here.  n == 0 gives scale 0 and no words.
 */
void orc_sign_ef_segment(int64_t n, const float* g, float* e, float* u, float m,
                         uint32_t* bits, float* scale_out)
{
    for (int64_t i = 0; i < n; ++i) {
        float x = g[i];
        if (u) {
            float mu = m * u[i];
            u[i] = mu + x;
            x = u[i];
        }
        e[i] = e[i] + x;
    }
    double s = 0.0;
    for (int64_t i = 0; i < n; ++i) s += fabs((double)e[i]);
    float scale = n > 0 ? (float)(s / (double)n) : 0.0f;
    *scale_out = scale;
    for (int64_t w = 0; w < (n + 31) / 32; ++w) bits[w] = 0;
    for (int64_t i = 0; i < n; ++i) {
        int neg = e[i] < 0.0f;
        if (neg) bits[i / 32] |= 1u << (i % 32);
        float q = neg ? -scale : scale;
        e[i] = e[i] - q;
    }
}

/* dense[i] = sign_i * scale (or += with accumulate) for one segment. */
void orc_sign_decompress_segment(int64_t n, const uint32_t* bits, float scale, float* dense,
                                 int accumulate)
{
    for (int64_t i = 0; i < n; ++i) {
        float v = ((bits[i / 32] >> (i % 32)) & 1u) ? -scale : scale;
        dense[i] = accumulate ? dense[i] + v : v;
    }
}

/* ------------------------------------------------------------ QSGD s-level codec */

/* Top 24 bits of the QSGD draw of global index gidx: word gidx % 4 of the Philox4x32-10
 * block at counter (gidx/4 lo, gidx/4 hi, step lo, 0x52) -- one block serves four
 * consecutive elements. */
static uint32_t qsgd_draw24(uint64_t seed, uint64_t step, int64_t gidx)
{
    uint64_t blk = (uint64_t)gidx >> 2;
    uint32_t ctr[4] = {(uint32_t)blk, (uint32_t)(blk >> 32), (uint32_t)step, 0x52u};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t r[4];
    orc_philox4x32_10(ctr, key, r);
    return r[(uint64_t)gidx & 3u] >> 8;
}

/*
 * QSGD with s levels ("Communication Optimization > Gradient Compression", QSGD paragraph:
 * Q_s(g) = ||g|| sgn(g) xi(g, s), xi rounding |g| / (||g|| / s) up or down at random so that
 * E[Q_s(g)] = g; at s = 2^b - 1 it is a b-bit code; the printed formula lacks the factor
 * 1/s that makes the expectation exact, restored here), one norm per segment.  With e (error
 * feedback, genomic-FL glossary quantization section) acc = e + x, else acc = x; x = g or
 * the momentum-corrected u.
 *   norm = fl32(sqrt(S)), S = sum acc_i^2 in double (index order);
 *   step = fl32(norm / s);  a = min(fl32(|acc| / step), s);  l = floor(a);
 *   xi = l + [u24 < (a - l) * 2^24]  (u24: top 24 bits of word (global index % 4) of the
 *        Philox4x32-10 block keyed (seed lo, seed hi) at counter (global index / 4 lo, hi,
 *        step lo, 0x52));
 *   code = sgn(acc) * xi (int8, |code| <= s <= 127); step == 0 gives code 0;
 *   with e: e = fl(acc - fl(code * step)).
 */
int orc_qsgd_segment(int64_t n, int64_t seg_base, const float* g, float* e, float* u, float m,
                     int32_t s, uint64_t seed, uint64_t step, int8_t* codes, float* norm_out)
{
    if (s < 1 || s > 127 || n < 0) return -1;
    float* acc = (float*)malloc((size_t)(n > 0 ? n : 1) * sizeof(float));
    if (!acc) return -1;
    for (int64_t i = 0; i < n; ++i) {
        float x = g[i];
        if (u) {
            float mu = m * u[i];
            u[i] = mu + x;
            x = u[i];
        }
        acc[i] = e ? e[i] + x : x;
    }
    double sq = 0.0;
    for (int64_t i = 0; i < n; ++i) sq += (double)acc[i] * (double)acc[i];
    float norm = (float)sqrt(sq);
    float qstep = norm / (float)s;
    *norm_out = norm;
    for (int64_t i = 0; i < n; ++i) {
        float v = acc[i];
        int q = 0;
        if (qstep != 0.0f) {
            float a = fabsf(v) / qstep;
            if (a > (float)s) a = (float)s;
            float l = floorf(a);
            float frac = a - l;
            q = (int)l + (((float)qsgd_draw24(seed, step, seg_base + i) < frac * 16777216.0f) ? 1 : 0);
        }
        int code = signbit(v) ? -q : q;
        codes[i] = (int8_t)code;
        if (e) {
            float deq = (float)code * qstep;
            e[i] = v - deq;
        }
    }
    free(acc);
    return 0;
}

/* dense[i] = fl(code_i * fl(norm / s)) (or += with accumulate). */
void orc_qsgd_decompress_segment(int64_t n, const int8_t* codes, float norm, int32_t s,
                                 float* dense, int accumulate)
{
    float qstep = norm / (float)s;
    for (int64_t i = 0; i < n; ++i) {
        float v = (float)codes[i] * qstep;
        dense[i] = accumulate ? dense[i] + v : v;
    }
}

/* ------------------------------------------------------------------- Random-k */

/* Random key of global index gidx: word gidx % 4 of the Philox4x32-10 block keyed (seed lo,
 * seed hi) at counter (gidx/4 lo, gidx/4 hi, step lo, 0x53), shifted right by one (31 bits). */
static uint32_t randk_key(uint64_t seed, uint64_t step, int64_t gidx)
{
    uint64_t blk = (uint64_t)gidx >> 2;
    uint32_t ctr[4] = {(uint32_t)blk, (uint32_t)(blk >> 32), (uint32_t)step, 0x53u};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t r[4];
    orc_philox4x32_10(ctr, key, r);
    return r[(uint64_t)gidx & 3u] >> 1;
}

/*
 * Random-k of one segment of n elements (global offset seg_base), k in [0, n]
 * (memory-compression glossary, Random-k section: a random mask per iteration, unbiased, no
 * sort of the gradient needed).  The mask is the k positions whose random keys are largest, equal keys
 * going to the lower position: sorting by independent uniform keys is a uniform random
 * permutation, so every k-subset is equally likely (up to the rare equal 31-bit keys).
 *   x = g, or with u the momentum-corrected u = fl(fl(m*u) + g);
 *   acc = fl(e + x) with e (error feedback), else acc = x;
 *   vals = acc at the mask in ascending index order, or without e fl(acc * fl32(n / k))
 *   (n / k formed in double, one rounding to float), whose expectation is acc;
 *   with e: e = +0 at the mask and acc elsewhere; mask_u zeroes u at the mask.
 */
int orc_randk_segment(int64_t n, int64_t k, int64_t seg_base, const float* g, float* e, float* u,
                      float m, int mask_u, uint64_t seed, uint64_t step, float* vals,
                      int32_t* idx)
{
    if (n < 0 || n > 0x7FFFFFFF || k < 0 || k > n) return -1;
    if (n == 0) return 0;
    float* acc = (float*)malloc((size_t)n * sizeof(float));
    rank_rec* rec = (rank_rec*)malloc((size_t)n * sizeof *rec);
    uint32_t* sel = (uint32_t*)malloc((size_t)(k > 0 ? k : 1) * sizeof *sel);
    if (!acc || !rec || !sel) { free(acc); free(rec); free(sel); return -1; }
    for (int64_t i = 0; i < n; ++i) {
        float x = g[i];
        if (u) {
            float mu = m * u[i];
            u[i] = mu + x;
            x = u[i];
        }
        acc[i] = e ? e[i] + x : x;
        rec[i].key = randk_key(seed, step, seg_base + i);
        rec[i].pos = (uint32_t)i;
    }
    qsort(rec, (size_t)n, sizeof *rec, by_rank);
    for (int64_t j = 0; j < k; ++j) sel[j] = rec[j].pos;
    free(rec);
    qsort(sel, (size_t)k, sizeof *sel, by_pos);
    float scale = k > 0 ? (float)((double)n / (double)k) : 0.0f;
    for (int64_t j = 0; j < k; ++j) {
        float v = acc[sel[j]];
        vals[j] = e ? v : v * scale;
        idx[j] = (int32_t)sel[j];
    }
    if (e) {
        for (int64_t i = 0; i < n; ++i) e[i] = acc[i];
        for (int64_t j = 0; j < k; ++j) e[sel[j]] = 0.0f;
    }
    if (u && mask_u)
        for (int64_t j = 0; j < k; ++j) u[sel[j]] = 0.0f;
    free(acc);
    free(sel);
    return 0;
}

/* -------------------------------------------------------------- gradient clipping */

/*
 * Local gradient clipping of one segment (genomic-FL glossary, DGC section; memory-compression
 * glossary, quantization section), the l2 reading: S = sum g_i^2 in double (index order),
 * norm = fl32(sqrt(S)); when norm > c, f = fl32(c / norm) and g_i = fl(g_i * f) in place;
 * otherwise g is left as it is.  *norm_out gets the norm before clipping.  c >= 0.
 */
void orc_clip_by_norm_segment(int64_t n, float* g, float c, float* norm_out)
{
    double sq = 0.0;
    for (int64_t i = 0; i < n; ++i) sq += (double)g[i] * (double)g[i];
    float norm = (float)sqrt(sq);
    *norm_out = norm;
    if (norm > c) {
        float f = c / norm;
        for (int64_t i = 0; i < n; ++i) g[i] = g[i] * f;
    }
}
