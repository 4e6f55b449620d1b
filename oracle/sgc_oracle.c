/*
 * sgc_oracle.c -- plain, slow, single-threaded CPU oracle of the per-step
 * sparse-gradient compression path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or
 * load this file; only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark do.  It shares no code, header, table or constant generator
 * with the HIP library: every rule below is written out again from the pages.
 *
 * Each function computes the plain definition of its step (a full sort for
 * exact top-k, bit-by-bit Rice coding, sequential sums); no blocking, fusion
 * or reordering beyond what the definition states.  fp32 arithmetic is plain
 * scalar C float arithmetic (x86-64 SSE, round-to-nearest-even, no fused
 * multiply-add: build with -ffp-contract=off); means are accumulated in
 * double precision.  Calls on distinct arrays may run in parallel threads:
 * the one file-scope variable (the array a qsort comparator reads) is
 * thread-local.
 *
 * Citations (page title, then section):
 *   [AH17]  "Sparse Communication for Distributed Gradient Descent"
 *           (Aji & Heafield, EMNLP 2017)
 *   [AHB19] "Combining Global Sparse Gradients with Local Gradients in
 *           Distributed Neural Network Training" (Aji, Heafield & Bogoychev,
 *           EMNLP-IJCNLP 2019)
 *   [SBC]   "Sparse Binary Compression: Towards Distributed Deep Learning
 *           with minimal Communication" (Sattler et al., arXiv 1805.08768)
 *
 * Where the pages leave a step open, the reading taken is stated at the step.
 *
 * The sampled-threshold mode (orc_sample_count, orc_compress_sampled)
 * follows a reading: the page that would define its sample is cut short.
 * Its sample size, sample positions and threshold are pinned by literal
 * examples worked out by hand from that reading.  Parity unpinned: in the
 * global+local combination, the reading that the local node's own sparse
 * message is summed as well as its dense gradient (pinned by linearity
 * only).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_EINVAL (-1)
#define ORC_ENOSPC (-2)

#define ORC_STATUS_TRUNCATED 1u
#define ORC_STATUS_CORRUPT 2u

#define ORC_GLOBAL 0
#define ORC_PER_SEGMENT 1

#define ORC_BIN_SBC 0
#define ORC_BIN_2BIT 1

/* Value source of one received message. */
#define ORC_VAL_F32 0   /* one fp32 value per entry */
#define ORC_VAL_SBC 1   /* one signed mean per segment */
#define ORC_VAL_2BIT 2  /* one 2-bit code per entry, two means per segment */

/* Codes per chunk-table entry of a Rice stream. */
#define ORC_CHUNK_CODES 256

/* ------------------------------------------------------------------------ */
/* Keep count.  [AH17] Abstract: the smallest 99% of updates by absolute
 * value are mapped to zero; [SBC] §II Sparse Binarization: the largest-
 * magnitude fraction p is retained.  Reading: k = ceil(n * ppm / 1e6) in
 * exact integer arithmetic (ppm = kept parts per million), at most n.      */
int64_t orc_keep_count(int64_t n, uint32_t ppm)
{
    if (n <= 0) return 0;
    int64_t k = (n * (int64_t)ppm + 999999) / 1000000;
    return k > n ? n : k;
}

/* Sample size of the sampled-threshold mode: min(n, max(smin, ceil(n/div))).
 * The sampling rule itself is a reading (the page that would define it is
 * cut short): systematic sampling, see orc_compress_sampled.               */
int64_t orc_sample_count(int64_t n, uint32_t sample_div, uint32_t sample_min)
{
    if (n <= 0) return 0;
    int64_t s = (n + (int64_t)sample_div - 1) / (int64_t)sample_div;
    if (s < (int64_t)sample_min) s = (int64_t)sample_min;
    return s > n ? n : s;
}

/* Warm-up schedule.  [SBC] appendix A (Warm-up Training): the kept fraction
 * falls exponentially, from 25% to 0.1%, over the first epochs.  Reading:
 * over `steps` steps the kept fraction moves geometrically from start to
 * end, p(t) = exp((1 - u) ln start + u ln end) with u = t / (steps - 1),
 * rounded to the nearest part per million; from the last warm-up step on
 * it stays at end.  Returns -1 on bad arguments.                           */
int64_t orc_warmup_ppm(int64_t t, int64_t steps, uint32_t start, uint32_t end)
{
    if (t < 0 || steps < 1 || start == 0 || end == 0 || start > 1000000 || end > 1000000) return -1;
    if (t == 0 && steps > 1) return start;
    if (t >= steps - 1) return end;
    double u = (double)t / (double)(steps - 1);
    double p = exp((1.0 - u) * log((double)start) + u * log((double)end));
    return (int64_t)floor(p + 0.5);
}

/* ------------------------------------------------------------------------ */
/* Rice code length statistics.  [SBC] §II Optimal Position Encoding: the
 * distances between nonzero elements are Golomb coded.  For a position set
 * in which every element is nonzero independently with probability p, the
 * gap z before a nonzero is geometric: P(z) = (1-p)^z p.  A Rice code with
 * parameter b spends b + 1 + floor(z / 2^b) bits on z, so its mean length is
 * b + 1 + sum_{j>=1} P(z >= j 2^b) = b + 1 + q/(1-q) with q = (1-p)^(2^b),
 * i.e. b + 1/(1 - (1-p)^(2^b)).                                              */
double orc_rice_expected_bits(int32_t b, double p)
{
    double q = pow(1.0 - p, ldexp(1.0, b));
    return (double)b + 1.0 / (1.0 - q);
}

/* The Rice parameter with the least mean length (ties to the smaller b).   */
int32_t orc_rice_param(double p)
{
    int32_t best = 0;
    double best_bits = orc_rice_expected_bits(0, p);
    for (int32_t b = 1; b <= 30; ++b) {
        double e = orc_rice_expected_bits(b, p);
        if (e < best_bits) { best = b; best_bits = e; }
    }
    return best;
}

/* ------------------------------------------------------------------------ */
static size_t alloc_n(int64_t n) { return n > 0 ? (size_t)n : 1u; }

static int all_finite(const float* x, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        if (!isfinite(x[i])) return 0;
    return 1;
}

static int valid_segments(const int64_t* seg_off, int32_t nseg)
{
    if (nseg < 1 || seg_off == NULL || seg_off[0] != 0) return 0;
    for (int32_t t = 0; t < nseg; ++t)
        if (seg_off[t + 1] < seg_off[t]) return 0;
    return seg_off[nseg] < ((int64_t)1 << 31);
}

/* Communication delay.  [SBC] §II Communication Delay: clients run several
 * local iterations before they exchange.  Between exchanges the fresh
 * gradient is only added to the carried residual: r <- fp32(r + g).        */
void orc_accumulate(const float* g, float* r, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) r[i] = r[i] + g[i];
}

/* Momentum correction.  [SBC] appendix A (Momentum Correction, Warm-up
 * Training and Momentum Masking): the momentum-corrected gradient, not the
 * raw gradient, is what goes into the residual.  The page gives neither the
 * momentum coefficient nor the update order; the reading taken: the local
 * momentum is updated first, u <- fp32(fp32(beta * u) + g), and the compress
 * step then adds u to the residual in place of g.                         */
void orc_momentum_correct(float beta, const float* g, float* u, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) {
        const float bu = beta * u[i];
        u[i] = bu + g[i];
    }
}

/* Momentum masking.  [SBC] appendix A: the momentum of the weights that were
 * updated is set to zero, so that stale momentum does not keep pushing them.
 * Reading: "updated" = sent; the entry becomes +0.                         */
void orc_momentum_mask(float* u, const int32_t* sent_idx, int64_t count)
{
    for (int64_t j = 0; j < count; ++j) u[sent_idx[j]] = 0.0f;
}

/* Order of the exact selection: larger |acc| first; among equal magnitudes
 * the lower index first (so the lower index wins a tie at the threshold).   */
static _Thread_local const float* sort_acc;
static int by_magnitude_then_index(const void* a, const void* b)
{
    int32_t i = *(const int32_t*)a, j = *(const int32_t*)b;
    float mi = fabsf(sort_acc[i]), mj = fabsf(sort_acc[j]);
    if (mi > mj) return -1;
    if (mi < mj) return 1;
    return (i < j) ? -1 : (i > j);
}

static int by_value_descending(const void* a, const void* b)
{
    float x = *(const float*)a, y = *(const float*)b;
    return (x > y) ? -1 : (x < y);
}

/* Emit the kept set ascending by global index, write the residual and the
 * per-segment counts.  Entries beyond cap are not sent and stay in the
 * residual.  Returns the number of kept elements that did not fit.        */
static int64_t emit_kept(const float* acc, const unsigned char* kept, float* r,
                         const int64_t* seg_off, int32_t nseg,
                         int32_t* out_idx, float* out_val, int64_t cap,
                         int64_t* out_counts)
{
    int64_t n = seg_off[nseg], total = 0, dropped = 0;
    for (int32_t t = 0; t <= nseg; ++t) out_counts[t] = 0;
    int32_t t = 0;
    for (int64_t i = 0; i < n; ++i) {
        while (i >= seg_off[t + 1]) ++t;
        if (kept[i] && total < cap) {
            out_idx[total] = (int32_t)i;
            out_val[total] = acc[i];
            ++total;
            ++out_counts[t];
            /* Residual accumulation ([SBC] §II Residual Accumulation): what is
             * sent leaves the residual.  Reading: the sent entry becomes +0. */
            r[i] = 0.0f;
        } else {
            if (kept[i]) ++dropped;
            r[i] = acc[i];
        }
    }
    out_counts[nseg] = total;
    return dropped;
}

/* Exact top-k compress step.
 * acc = fp32(r + g) ([SBC] §II Residual Accumulation: the residual is added
 * to the new update); per selection group the k = keep_count(m, ppm) entries
 * of largest |acc| are kept, lower index first among equal magnitudes
 * ([AH17] Abstract: the smallest 99% by absolute value become zero); kept
 * (index, value) pairs are emitted ascending ([AH17] Abstract: sparse
 * matrices are exchanged) and zeroed in the residual.  scope = ORC_GLOBAL
 * selects over the whole vector (segments concatenated in order), or
 * ORC_PER_SEGMENT selects within each segment.
 * Returns the number of emitted entries, or a negative error code.        */
int64_t orc_compress_exact(const float* g, float* r, const int64_t* seg_off,
                           int32_t nseg, int32_t scope, uint32_t ppm,
                           int32_t* out_idx, float* out_val, int64_t cap,
                           int64_t* out_counts)
{
    if (!valid_segments(seg_off, nseg) || ppm > 1000000) return ORC_EINVAL;
    int64_t n = seg_off[nseg];
    if (!all_finite(g, n) || !all_finite(r, n)) return ORC_EINVAL;
    float* acc = (float*)malloc(alloc_n(n) * sizeof(float));
    unsigned char* kept = (unsigned char*)calloc(alloc_n(n), 1);
    int32_t* order = (int32_t*)malloc(alloc_n(n) * sizeof(int32_t));
    if (!acc || !kept || !order) { free(acc); free(kept); free(order); return ORC_ENOSPC; }

    for (int64_t i = 0; i < n; ++i) acc[i] = r[i] + g[i];

    int32_t ngroups = (scope == ORC_GLOBAL) ? 1 : nseg;
    int64_t need = 0;
    for (int32_t gi = 0; gi < ngroups; ++gi) {
        int64_t lo = (scope == ORC_GLOBAL) ? 0 : seg_off[gi];
        int64_t hi = (scope == ORC_GLOBAL) ? n : seg_off[gi + 1];
        int64_t m = hi - lo, k = orc_keep_count(m, ppm);
        need += k;
        for (int64_t j = 0; j < m; ++j) order[j] = (int32_t)(lo + j);
        sort_acc = acc;
        qsort(order, (size_t)m, sizeof(int32_t), by_magnitude_then_index);
        for (int64_t j = 0; j < k; ++j) kept[order[j]] = 1;
    }
    if (need > cap) { free(acc); free(kept); free(order); return ORC_ENOSPC; }
    emit_kept(acc, kept, r, seg_off, nseg, out_idx, out_val, cap, out_counts);
    free(acc); free(kept); free(order);
    return out_counts[nseg];
}

/* Sampled-threshold compress step (the threshold-estimation variant).
 * Per selection group of m elements: s = sample_count(m) systematic sample
 * positions lo + floor((2j+1) m / (2s)), j = 0..s-1; T = the ks-th largest
 * sampled |acc| with ks = keep_count(s, ppm); every element with |acc| >= T
 * is kept (so all ties at T are kept).  If more than cap are kept overall,
 * the first cap in index order are sent, the rest stay in the residual and
 * ORC_STATUS_TRUNCATED is set.  Returns the number emitted or an error.    */
int64_t orc_compress_sampled(const float* g, float* r, const int64_t* seg_off,
                             int32_t nseg, int32_t scope, uint32_t ppm,
                             uint32_t sample_div, uint32_t sample_min,
                             int32_t* out_idx, float* out_val, int64_t cap,
                             int64_t* out_counts, uint32_t* status)
{
    if (!valid_segments(seg_off, nseg) || ppm > 1000000 || sample_div == 0) return ORC_EINVAL;
    int64_t n = seg_off[nseg];
    if (!all_finite(g, n) || !all_finite(r, n)) return ORC_EINVAL;
    float* acc = (float*)malloc(alloc_n(n) * sizeof(float));
    unsigned char* kept = (unsigned char*)calloc(alloc_n(n), 1);
    float* mags = (float*)malloc(alloc_n(n) * sizeof(float));
    if (!acc || !kept || !mags) { free(acc); free(kept); free(mags); return ORC_ENOSPC; }

    for (int64_t i = 0; i < n; ++i) acc[i] = r[i] + g[i];

    int32_t ngroups = (scope == ORC_GLOBAL) ? 1 : nseg;
    for (int32_t gi = 0; gi < ngroups; ++gi) {
        int64_t lo = (scope == ORC_GLOBAL) ? 0 : seg_off[gi];
        int64_t hi = (scope == ORC_GLOBAL) ? n : seg_off[gi + 1];
        int64_t m = hi - lo;
        if (m == 0) continue;
        int64_t s = orc_sample_count(m, sample_div, sample_min);
        for (int64_t j = 0; j < s; ++j) {
            uint64_t pos = ((uint64_t)(2 * j + 1) * (uint64_t)m) / (uint64_t)(2 * s);
            mags[j] = fabsf(acc[lo + (int64_t)pos]);
        }
        qsort(mags, (size_t)s, sizeof(float), by_value_descending);
        int64_t ks = orc_keep_count(s, ppm);
        if (ks == 0) continue;
        float thr = mags[ks - 1];
        for (int64_t i = lo; i < hi; ++i)
            if (fabsf(acc[i]) >= thr) kept[i] = 1;
    }
    int64_t dropped = emit_kept(acc, kept, r, seg_off, nseg, out_idx, out_val, cap, out_counts);
    if (status && dropped > 0) *status |= ORC_STATUS_TRUNCATED;
    free(acc); free(kept); free(mags);
    return out_counts[nseg];
}

/* ------------------------------------------------------------------------ */
/* Binarize the kept values of every segment.
 * [SBC] §II Sparse Binarization: after top-p selection by magnitude, the
 * positive and the negative kept values are each summarised by their mean;
 * only the side whose mean has the larger absolute value stays nonzero and
 * is sent as that one mean.  [SBC] appendix C: the projection onto the
 * subspace is unique -- the mean is the least-squares single value of the
 * side.  [SBC] §II Residual Accumulation: what is not sent stays in the
 * residual.
 * Readings: sums in double in ascending index order; mu = fp32(S/c), 0 if
 * the side is empty; the positive side wins a tie of the fp32 means; zeros
 * are in neither side and never sent; the residual of an entry becomes
 * fp32(v - sent value) (v itself if unsent).
 * ORC_BIN_2BIT (the quantization that [AH17] Abstract combines with
 * dropping; the page is cut before its definition): every kept value is
 * replaced by +mu_pos (code 1), -mu_neg (code 2) or +0 (code 0, v = +-0);
 * codes are 2 bits, LSB-first, 16 per 32-bit word; means[2t] = +mu_pos,
 * means[2t+1] = -mu_neg.  For SBC, means[t] is the signed mean sent.
 * Returns the number of entries in the output message.                    */
int64_t orc_binarize(const int32_t* idx, const float* val, const int64_t* counts,
                     int32_t nseg, int32_t mode, float* r,
                     int32_t* out_idx, int64_t* out_counts, float* out_means,
                     uint32_t* out_codes)
{
    if (nseg < 1 || (mode != ORC_BIN_SBC && mode != ORC_BIN_2BIT)) return ORC_EINVAL;
    int64_t total_in = counts[nseg], e0 = 0, total_out = 0;
    if (mode == ORC_BIN_2BIT)
        for (int64_t w = 0; w < (total_in + 15) / 16; ++w) out_codes[w] = 0;
    for (int32_t t = 0; t < nseg; ++t) {
        int64_t e1 = e0 + counts[t];
        int64_t cp = 0, cn = 0;
        double sp = 0.0, sn = 0.0;
        for (int64_t j = e0; j < e1; ++j) {
            float v = val[j];
            if (v > 0.0f) { ++cp; sp += (double)v; }
            else if (v < 0.0f) { ++cn; sn += -(double)v; }
        }
        float mu_pos = cp ? (float)(sp / (double)cp) : 0.0f;
        float mu_neg = cn ? (float)(sn / (double)cn) : 0.0f;
        if (mode == ORC_BIN_SBC) {
            int64_t sent = 0;
            float mean = 0.0f;
            if (cp + cn > 0) {
                int positive = mu_pos >= mu_neg;
                mean = positive ? mu_pos : -mu_neg;
                for (int64_t j = e0; j < e1; ++j) {
                    float v = val[j];
                    if ((positive && v > 0.0f) || (!positive && v < 0.0f)) {
                        out_idx[total_out + sent] = idx[j];
                        ++sent;
                        r[idx[j]] = v - mean;
                    } else {
                        r[idx[j]] = v;
                    }
                }
            } else {
                for (int64_t j = e0; j < e1; ++j) r[idx[j]] = val[j];
            }
            out_means[t] = mean;
            out_counts[t] = sent;
            total_out += sent;
        } else {
            out_means[2 * t] = mu_pos;
            out_means[2 * t + 1] = -mu_neg;
            for (int64_t j = e0; j < e1; ++j) {
                float v = val[j];
                uint32_t code = (v > 0.0f) ? 1u : (v < 0.0f) ? 2u : 0u;
                float q = (code == 1u) ? mu_pos : (code == 2u) ? -mu_neg : 0.0f;
                r[idx[j]] = v - q;
                out_codes[j / 16] |= code << (2 * (j % 16));
                out_idx[j] = idx[j];
            }
            out_counts[t] = counts[t];
            total_out += counts[t];
        }
        e0 = e1;
    }
    out_counts[nseg] = total_out;
    return total_out;
}

/* ------------------------------------------------------------------------ */
/* Rice/Golomb position encoding.  [SBC] §II Optimal Position Encoding: the
 * distances between nonzero elements are sent instead of the positions;
 * [SBC] appendix A: the decoder needs no shape information because both
 * ends know every tensor shape.
 * A stream is the whole vector (ORC_GLOBAL, positions = global indices) or
 * one segment (ORC_PER_SEGMENT, positions relative to the segment start).
 * Readings: the coded gap is z = pos - prev - 1 (prev = -1 before the first
 * entry), i.e. the number of zeros skipped; the code of z is floor(z / 2^b)
 * one-bits, one zero-bit, then the b low bits of z least-significant first;
 * stream bit i is bit (i mod 32) of word i/32 of the stream; each stream
 * starts on a word boundary and its pad bits are 0; the chunk table holds,
 * for codes 0, C, 2C, ... (C = 256) of every stream, two entries: the
 * stream-relative bit offset of the code and the stream-relative position
 * reached before it (previous position + 1, 0 for code 0), so that a
 * decoder can start in the middle of a stream.  chunk_cap counts entries.
 * Returns ORC_OK, ORC_EINVAL (indices not strictly ascending or out of the
 * stream) or ORC_ENOSPC (word_cap or chunk_cap too small).                */
struct bitwriter { uint32_t* words; int64_t cap; int64_t base; uint64_t bit; int overflow; };

static void put_bit(struct bitwriter* w, unsigned v)
{
    int64_t wi = w->base + (int64_t)(w->bit >> 5);
    if (wi >= w->cap) { w->overflow = 1; }
    else if (v) w->words[wi] |= 1u << (w->bit & 31);
    w->bit++;
}

int32_t orc_encode(const int32_t* idx, const int64_t* counts, const int64_t* seg_off,
                   int32_t nseg, int32_t scope, int32_t b,
                   uint32_t* words, int64_t word_cap, uint64_t* word_off,
                   uint64_t* nbits, uint64_t* chunk_off, int64_t chunk_cap)
{
    if (!valid_segments(seg_off, nseg) || b < 0 || b > 30) return ORC_EINVAL;
    for (int64_t i = 0; i < word_cap; ++i) words[i] = 0;
    int32_t nstreams = (scope == ORC_GLOBAL) ? 1 : nseg;
    int64_t e0 = 0, word_pos = 0, chunk_pos = 0;
    for (int32_t s = 0; s < nstreams; ++s) {
        int64_t cnt = (scope == ORC_GLOBAL) ? counts[nseg] : counts[s];
        int64_t lo = (scope == ORC_GLOBAL) ? 0 : seg_off[s];
        int64_t hi = (scope == ORC_GLOBAL) ? seg_off[nseg] : seg_off[s + 1];
        struct bitwriter w = { words, word_cap, word_pos, 0, 0 };
        int64_t prev = -1;
        word_off[s] = (uint64_t)word_pos;
        for (int64_t q = 0; q < cnt; ++q) {
            if (q % ORC_CHUNK_CODES == 0) {
                if (chunk_pos + 2 > chunk_cap) return ORC_ENOSPC;
                chunk_off[chunk_pos++] = w.bit;
                chunk_off[chunk_pos++] = (uint64_t)(prev + 1);
            }
            int64_t pos = (int64_t)idx[e0 + q] - lo;
            if (pos <= prev || pos >= hi - lo) return ORC_EINVAL;
            uint64_t z = (uint64_t)(pos - prev - 1);
            prev = pos;
            for (uint64_t u = 0; u < (z >> b); ++u) put_bit(&w, 1);
            put_bit(&w, 0);
            for (int32_t i = 0; i < b; ++i) put_bit(&w, (unsigned)((z >> i) & 1u));
        }
        if (w.overflow) return ORC_ENOSPC;
        nbits[s] = w.bit;
        word_pos += (int64_t)((w.bit + 31) / 32);
        e0 += cnt;
    }
    word_off[nstreams] = (uint64_t)word_pos;
    return ORC_OK;
}

/* Decode the positions of one Rice stream (the inverse of orc_encode).
 * Reads count codes starting at words[0]; pos = prev + 1 + z.  Sets
 * ORC_STATUS_CORRUPT in *status if a read passes nbits, a position reaches
 * numel, a chunk-table entry (bit offset, position reached) disagrees with
 * the decoded stream, or the codes do not use exactly nbits bits.
 * Positions are stream-relative.                                          */
int32_t orc_decode_stream(const uint32_t* words, uint64_t nbits, int64_t count,
                          int32_t b, int64_t numel, const uint64_t* chunk_off,
                          int64_t* out_pos, uint32_t* status)
{
    uint64_t bit = 0;
    int64_t prev = -1;
    for (int64_t q = 0; q < count; ++q) {
        if (chunk_off && q % ORC_CHUNK_CODES == 0 &&
            (chunk_off[2 * (q / ORC_CHUNK_CODES)] != bit ||
             chunk_off[2 * (q / ORC_CHUNK_CODES) + 1] != (uint64_t)(prev + 1))) {
            *status |= ORC_STATUS_CORRUPT;
            return ORC_OK;
        }
        uint64_t ones = 0;
        for (;;) {
            if (bit >= nbits) { *status |= ORC_STATUS_CORRUPT; return ORC_OK; }
            unsigned v = (words[bit >> 5] >> (bit & 31)) & 1u;
            ++bit;
            if (!v) break;
            ++ones;
        }
        uint64_t rem = 0;
        for (int32_t i = 0; i < b; ++i) {
            if (bit >= nbits) { *status |= ORC_STATUS_CORRUPT; return ORC_OK; }
            rem |= (uint64_t)((words[bit >> 5] >> (bit & 31)) & 1u) << i;
            ++bit;
        }
        uint64_t z = ones * ((uint64_t)1 << b) + rem;
        if (z >= (uint64_t)numel) { *status |= ORC_STATUS_CORRUPT; return ORC_OK; }
        int64_t pos = prev + 1 + (int64_t)z;
        if (pos >= numel) { *status |= ORC_STATUS_CORRUPT; return ORC_OK; }
        out_pos[q] = pos;
        prev = pos;
    }
    if (bit != nbits) *status |= ORC_STATUS_CORRUPT;
    return ORC_OK;
}

/* Add one received message into the dense buffer.
 * [SBC] §I: the clients' updates are combined by a central server or an
 * all-reduce; [AHB19] Abstract: the compressed global gradient may be
 * combined with the node's own uncompressed local gradient (the caller sets
 * the dense buffer to that local gradient before the first message).
 * Readings: updates are summed (no 1/W); messages are applied in the order
 * the caller calls this function; only entries present in the message are
 * added, out[pos] <- fp32(out[pos] + value).
 * Positions come from idx (raw messages, golomb == 0) or from decoding the
 * Rice streams (golomb != 0, streams laid out as orc_encode writes them).
 * Values: vkind ORC_VAL_F32 -> val[j]; ORC_VAL_SBC -> means[t] of the entry's
 * segment t; ORC_VAL_2BIT -> code c of entry j: 0 -> +0, 1 -> means[2t],
 * 2 -> means[2t+1], 3 -> corrupt.  The segment of an entry is given by the
 * per-segment counts (entries are ascending).                              */
int32_t orc_accumulate_message(float* out, const int64_t* seg_off, int32_t nseg,
                               int32_t golomb, int32_t scope, int32_t b,
                               int32_t vkind, const int64_t* counts,
                               const int32_t* idx, const float* val,
                               const uint32_t* codes, const float* means,
                               const uint32_t* words, const uint64_t* word_off,
                               const uint64_t* nbits, const uint64_t* chunk_off,
                               uint32_t* status)
{
    if (!valid_segments(seg_off, nseg)) return ORC_EINVAL;
    int64_t n = seg_off[nseg], total = counts[nseg];
    int64_t* pos = (int64_t*)malloc(alloc_n(total) * sizeof(int64_t));
    if (!pos) return ORC_ENOSPC;
    uint32_t st = 0;
    if (!golomb) {
        for (int64_t j = 0; j < total; ++j) {
            pos[j] = idx[j];
            if (idx[j] < 0 || idx[j] >= n) st |= ORC_STATUS_CORRUPT;
        }
    } else if (scope == ORC_GLOBAL) {
        orc_decode_stream(words + word_off[0], nbits[0], total, b, n, chunk_off, pos, &st);
    } else {
        int64_t e0 = 0, c0 = 0;
        for (int32_t t = 0; t < nseg && !st; ++t) {
            int64_t numel = seg_off[t + 1] - seg_off[t];
            orc_decode_stream(words + word_off[t], nbits[t], counts[t], b, numel,
                              chunk_off ? chunk_off + c0 : NULL, pos + e0, &st);
            for (int64_t j = e0; j < e0 + counts[t]; ++j) pos[j] += seg_off[t];
            e0 += counts[t];
            c0 += 2 * ((counts[t] + ORC_CHUNK_CODES - 1) / ORC_CHUNK_CODES);
        }
    }
    if (!st && vkind == ORC_VAL_2BIT)
        for (int64_t j = 0; j < total; ++j)
            if (((codes[j / 16] >> (2 * (j % 16))) & 3u) == 3u) st |= ORC_STATUS_CORRUPT;
    if (st) {
        *status |= st;
        free(pos);
        return ORC_OK;
    }
    int64_t e0 = 0;
    for (int32_t t = 0; t < nseg; ++t) {
        for (int64_t j = e0; j < e0 + counts[t]; ++j) {
            float v;
            if (vkind == ORC_VAL_F32) v = val[j];
            else if (vkind == ORC_VAL_SBC) v = means[t];
            else {
                uint32_t c = (codes[j / 16] >> (2 * (j % 16))) & 3u;
                v = (c == 0u) ? 0.0f : (c == 1u) ? means[2 * t] : means[2 * t + 1];
            }
            out[pos[j]] = out[pos[j]] + v;
        }
        e0 += counts[t];
    }
    free(pos);
    return ORC_OK;
}
