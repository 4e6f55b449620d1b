/*
 * sgc.h -- C ABI of the MI355X (gfx950) sparse-gradient compression library.
 *
 * One training step of a data-parallel worker, as the pages describe it:
 * add the carried residual to the fresh fp32 gradient, keep only the
 * largest-magnitude fraction of the result, send those (index, value) pairs
 * and keep the rest as the new residual; optionally binarize or quantize the
 * kept values; optionally code the index gaps with a Rice (power-of-two
 * Golomb) code.  The receiver decodes several workers' messages and adds
 * them, in a fixed order, into a dense buffer that may start as the node's
 * own local gradient.
 *
 * Citations (page title, then section):
 *   [AH17]  "Sparse Communication for Distributed Gradient Descent"
 *           (Aji & Heafield, EMNLP 2017)
 *   [AHB19] "Combining Global Sparse Gradients with Local Gradients in
 *           Distributed Neural Network Training" (Aji, Heafield & Bogoychev)
 *   [SBC]   "Sparse Binary Compression: Towards Distributed Deep Learning
 *           with minimal Communication" (Sattler et al., arXiv 1805.08768)
 *
 * Conventions shared by every call
 * --------------------------------
 * - A *layout* describes the flat parameter vector as nseg contiguous
 *   segments (one per tensor, in order) with n = sum of their sizes < 2^31.
 *   [SBC] appendix A: both ends know every tensor shape, so messages carry
 *   no shape information; the layout is that shared knowledge.
 * - Every data pointer is caller-owned DEVICE memory on the device that is
 *   current when the call is made; fp32 gradient/residual/output buffers
 *   must be 16-byte aligned.  Option structs, message descriptors and other
 *   arguments marked [host] are read during the call only.
 * - Calls are asynchronous on `stream` (a hipStream_t, NULL = the default
 *   stream).  Outputs are valid once the stream reaches the call.  The
 *   library never allocates device memory on these calls: scratch space is
 *   the caller's `ws`, at least the size the matching *_workspace call
 *   returns.  Calls that may overlap in time need distinct workspaces.
 * - Every argument check is done on the host before any GPU work is queued
 *   and is reported by the return code (SGC_E*).  Conditions only the
 *   device can see are OR-ed into *dstatus (device uint32, may be NULL).
 * - Results are deterministic: no floating-point atomics; every sum has a
 *   fixed order.
 * - A layout's tables are put on a device once, at set-up, by
 *   sgc_layout_upload; the compute calls then queue only kernel launches on
 *   `stream` -- no allocation, memset or synchronous copy -- so a sequence
 *   of calls can be captured into a HIP graph and replayed.  A compute call
 *   on a device the layout was not uploaded to returns SGC_ENOTREADY.  The
 *   sgc_layout_* calls cannot be captured.
 */
#ifndef SGC_H
#define SGC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SGC_ABI_VERSION 3

/* Return codes. */
#define SGC_OK 0
#define SGC_EINVAL (-1)       /* bad argument: null pointer, misaligned buffer, bad layout, cap too small */
#define SGC_ENOSPC (-2)       /* workspace or an output capacity below the host-computable bound */
#define SGC_EHIP (-3)         /* a HIP runtime call or kernel launch failed */
#define SGC_EUNSUPPORTED (-4) /* valid but unsupported combination */
#define SGC_ENOTREADY (-5)    /* the layout was not uploaded to the current device */

/* Device status bits, OR-ed into *dstatus. */
#define SGC_STATUS_TRUNCATED 1u   /* sampled mode kept more than cap: the first cap (index order) were sent */
#define SGC_STATUS_CORRUPT 2u     /* a message failed to decode (that message is skipped entirely) */
#define SGC_STATUS_DENSE_PATH 4u  /* exact selection could not use its sampled bounds for a group: it was selected from all its candidates or the whole residual (informational, result unchanged) */
#define SGC_STATUS_BAD_INPUT 8u   /* encode: indices not strictly ascending inside a stream (output undefined) */

/* Compress modes. */
#define SGC_EXACT 0           /* exact top-k, lower index wins ties */
#define SGC_SAMPLED 1         /* threshold estimated from a systematic sample, every |acc| >= T kept */
#define SGC_ACCUMULATE_ONLY 2 /* communication delay: r <- r + g only */
#define SGC_HOLD_KEPT 0x10    /* flag for SGC_EXACT / SGC_SAMPLED: kept entries keep acc in the residual */

/* Compress pipelines (sgc_compress_opts.path); every choice gives the same
 * result bit for bit. */
#define SGC_PATH_AUTO 0u      /* window above about 2.5% kept or from 2^29 elements on, else gather */
#define SGC_PATH_GATHER 1u    /* candidates copied into one array, selected and compacted (fastest at low kept fractions) */
#define SGC_PATH_WINDOW 2u    /* only entries between the probe's bounds selected; output written from the tile regions */

/* Selection / stream scope. */
#define SGC_GLOBAL 0      /* one selection (one Rice stream) over the whole vector */
#define SGC_PER_SEGMENT 1 /* one selection (one Rice stream) per segment */

/* Binarize modes. */
#define SGC_BIN_SBC 0  /* sparse binarization: one signed mean per segment, one sign side sent */
#define SGC_BIN_2BIT 1 /* ternary 2-bit codes {0, +mean_pos, -mean_neg} per kept value */
#define SGC_BIN_HELD 0x10 /* flag: the residual holds acc (= val) at the kept entries, not +0 */

/* Received message formats. */
#define SGC_MSG_RAW_F32 0     /* idx[] + val[] */
#define SGC_MSG_RAW_2BIT 1    /* idx[] + 2-bit codes[] + means[2*nseg] */
#define SGC_MSG_GOLOMB_F32 2  /* Rice-coded positions + val[] */
#define SGC_MSG_GOLOMB_SBC 3  /* Rice-coded positions + means[nseg] */
#define SGC_MSG_GOLOMB_2BIT 4 /* Rice-coded positions + 2-bit codes[] + means[2*nseg] */

/* Initial contents of the dense output of decode-accumulate. */
#define SGC_INIT_ZERO 0    /* out = 0 */
#define SGC_INIT_BASE 1    /* out = base (e.g. the local dense gradient, [AHB19] Abstract) */
#define SGC_INIT_INPLACE 2 /* out keeps its contents */

/* Codes per chunk-table entry of a Rice stream. */
#define SGC_CHUNK_CODES 256

typedef void* sgc_stream_t; /* hipStream_t */

/* ------------------------------------------------------------------------
 * Layout.  seg_numel [host, nseg entries >= 0]; n = sum < 2^31; nseg >= 1.
 * Creation checks the table and keeps a host copy.  Returns SGC_EINVAL on a
 * bad table, SGC_ENOSPC if host memory runs out.
 * sgc_layout_upload puts the tables on the current device (set-up, not the
 * hot path: one small hipMalloc and a synchronous copy; a repeated call on
 * the same device returns SGC_OK at once).  Every compute call needs it
 * done on its device first.  SGC_EINVAL for a NULL layout, SGC_EHIP if the
 * allocation or the copy fails.
 * sgc_layout_destroy frees the host copy and every device copy; no call
 * using the layout may still be in flight.  A layout is immutable once
 * uploaded and may be shared across threads.                               */
typedef struct sgc_layout sgc_layout;
int sgc_layout_create(const int64_t* seg_numel, int32_t nseg, sgc_layout** out);
int sgc_layout_upload(sgc_layout* layout);
void sgc_layout_destroy(sgc_layout* layout);
int64_t sgc_layout_numel(const sgc_layout* layout);
int32_t sgc_layout_nseg(const sgc_layout* layout);

/* ------------------------------------------------------------------------
 * Host helpers.
 * sgc_keep_count: entries kept out of n at keep_ppm kept parts per million,
 *   ceil(n * keep_ppm / 1e6) in integers, at most n ([AH17] Abstract: the
 *   smallest 99% by absolute value are dropped; [SBC] §II Sparse
 *   Binarization: the largest fraction p is kept).  -1 on bad arguments.
 * sgc_rice_param: the Rice parameter b minimising the mean code length
 *   b + 1/(1 - (1-p)^(2^b)) of geometric gaps at density p, ties to the
 *   smaller b ([SBC] §II Optimal Position Encoding).  -1 unless 0 < p <= 1.
 * sgc_warmup_ppm: the kept parts per million of step `step` (0-based) of a
 *   warm-up of `steps` steps whose kept fraction falls exponentially from
 *   start_ppm to end_ppm ([SBC] appendix A, Warm-up Training: from 25% to
 *   0.1% over the first epochs): start * (end/start)^(step/(steps-1))
 *   rounded to the nearest integer, start_ppm at step 0 and end_ppm from
 *   step steps-1 on.  -1 unless step >= 0, steps >= 1 and both fractions
 *   are in [1, 1e6].  The compress calls take any keep_ppm, so a caller
 *   runs the warm-up by passing this value at each step.                  */
int64_t sgc_keep_count(int64_t n, uint32_t keep_ppm);
int32_t sgc_rice_param(double p);
int64_t sgc_warmup_ppm(int64_t step, int64_t steps, uint32_t start_ppm, uint32_t end_ppm);
const char* sgc_strerror(int code);
int32_t sgc_abi_version(void);

/* ------------------------------------------------------------------------
 * Compress one step ([SBC] §II Residual Accumulation, Sparse Binarization;
 * [AH17] Abstract; [SBC] §II Communication Delay for SGC_ACCUMULATE_ONLY).
 *
 *   acc = fp32(residual + grad)                    (IEEE, round to nearest)
 *   SGC_EXACT:   per selection group (the vector, or each segment) keep the
 *                k = sgc_keep_count(m, keep_ppm) entries of largest |acc|,
 *                the lower index first among equal magnitudes.
 *   SGC_SAMPLED: per group of m elements take s = min(m, max(sample_min,
 *                ceil(m / sample_div))) systematic samples at positions
 *                floor((2j+1) m / (2s)); T = the ks-th largest sampled |acc|
 *                with ks = sgc_keep_count(s, keep_ppm); keep every |acc| >= T.
 *                If more than cap are kept the first cap in index order are
 *                sent and SGC_STATUS_TRUNCATED is set.
 *   Kept entries are written ascending by global index: out_idx (int32),
 *   out_val (the fp32 bits of acc); residual <- acc with kept entries +0.0.
 *   out_counts [device, nseg+1]: kept entries per segment (in both scopes),
 *   then the total.
 *   SGC_ACCUMULATE_ONLY: residual <- fp32(residual + grad); the out_*, ws
 *   and dstatus arguments are ignored and may be NULL.
 *   SGC_HOLD_KEPT (or-ed into SGC_EXACT or SGC_SAMPLED): the kept entries
 *   keep acc in the residual instead of +0; everything else is unchanged.
 *   For a caller that binarizes next (sgc_binarize with SGC_BIN_HELD), which
 *   then writes only the residual entries binarization changes -- half the
 *   scattered writes of the two calls without the flags.  Not accepted by
 *   sgc_compress_momentum (SGC_EUNSUPPORTED).
 *
 * grad [device, n fp32] is read; residual [device, n fp32] is updated in
 * place.  cap = capacity of out_idx/out_val; SGC_EXACT requires cap >= the
 * sum of the groups' k (else SGC_EINVAL).  keep_ppm <= 1e6, sample_div >= 1.
 * sgc_compress_workspace returns the ws bytes needed (0 on bad arguments),
 * which depends on the pipeline (opts.path) the call takes. */
typedef struct {
    int32_t mode;        /* SGC_EXACT | SGC_SAMPLED | SGC_ACCUMULATE_ONLY */
    int32_t scope;       /* SGC_GLOBAL | SGC_PER_SEGMENT */
    uint32_t keep_ppm;   /* kept parts per million: 10000 = top-1%, 1000 = top-0.1% */
    uint32_t sample_div; /* SGC_SAMPLED: sample one per sample_div elements (default 1000) */
    uint32_t sample_min; /* SGC_SAMPLED: at least this many samples per group (default 65536) */
    uint32_t path;       /* SGC_PATH_AUTO (0), SGC_PATH_GATHER or SGC_PATH_WINDOW: how the work is done, not what */
} sgc_compress_opts;

size_t sgc_compress_workspace(const sgc_layout* layout, const sgc_compress_opts* opt, int64_t cap);
int sgc_compress(const sgc_layout* layout, const sgc_compress_opts* opt,
                 const float* grad, float* residual,
                 int32_t* out_idx, float* out_val, int64_t cap, int64_t* out_counts,
                 uint32_t* dstatus, void* ws, size_t ws_bytes, sgc_stream_t stream);

/* ------------------------------------------------------------------------
 * Compress without allocating -- for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.
 *
 * Exactly sgc_compress (same arguments, results, status and errors), with
 * the library's own scratch buffer in place of ws: a file-scope device array
 * of SGC_NOALLOC_SCRATCH_BYTES that every GPU the library runs on holds from
 * its first layout upload until the process ends.  The call itself performs
 * no allocation of any kind.  Returns SGC_ENOSPC when the call would need
 * more workspace than that (sgc_compress_workspace(layout, opt, cap) >
 * SGC_NOALLOC_SCRATCH_BYTES: past about 77M elements at top-1% in one group,
 * 35M at top-10%),
 * SGC_ENOTREADY if no layout was uploaded to the current device (the upload
 * looks up the buffer's device address).  Every call on a GPU shares that
 * GPU's buffer, so calls that may overlap in time on one GPU (two streams,
 * two threads) race and give wrong results: serialise them.  The buffer
 * keeps the last call's contents; the compress kernels clear what they need
 * cleared themselves.                                                     */
#define SGC_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int sgc_compress_noalloc(const sgc_layout* layout, const sgc_compress_opts* opt,
                         const float* grad, float* residual,
                         int32_t* out_idx, float* out_val, int64_t cap, int64_t* out_counts,
                         uint32_t* dstatus, sgc_stream_t stream);

/* ------------------------------------------------------------------------
 * Compress one step with momentum correction and momentum masking ([SBC]
 * appendix A Momentum Correction, Warm-up Training and Momentum Masking:
 * the momentum-corrected gradient is added to the residual, and the
 * momentum of the updated weights is set to zero).  The page gives no
 * coefficient and no order; this call takes beta from the caller and
 * updates the momentum first:
 *
 *   u   = fp32(fp32(beta * momentum) + grad)       (two roundings, no FMA)
 *   then exactly sgc_compress with u in place of grad (acc = fp32(residual
 *   + u), the same selection, outputs, counts and status);
 *   momentum <- u, with +0.0 at every sent entry (entries kept but past cap
 *   in SGC_SAMPLED mode are not sent and keep u, like their residual).
 *   SGC_ACCUMULATE_ONLY: momentum <- u; residual <- fp32(residual + u).
 *
 * momentum [device, n fp32, 16-byte aligned] is updated in place; beta must
 * be finite (else SGC_EINVAL); other arguments and errors as sgc_compress.
 * The workspace is larger than sgc_compress's (candidates also carry u):
 * size it with sgc_compress_momentum_workspace.  beta = 0 gives
 * sgc_compress's selection with momentum <- grad (masked).               */
size_t sgc_compress_momentum_workspace(const sgc_layout* layout, const sgc_compress_opts* opt, int64_t cap);
int sgc_compress_momentum(const sgc_layout* layout, const sgc_compress_opts* opt, float beta,
                          const float* grad, float* momentum, float* residual,
                          int32_t* out_idx, float* out_val, int64_t cap, int64_t* out_counts,
                          uint32_t* dstatus, void* ws, size_t ws_bytes, sgc_stream_t stream);

/* ------------------------------------------------------------------------
 * Binarize the kept values of each segment ([SBC] §II Sparse Binarization;
 * [SBC] appendix C: the mean is the unique least-squares single value;
 * [AH17] Abstract: dropping combined with quantization).
 *
 * Input: a compress result (idx, val ascending; counts [device, nseg+1]);
 * cap >= counts[nseg] is the capacity the host sizes with.  Per segment
 * the positive and negative kept values are summed in double precision;
 * mean_pos = fp32(S_pos / c_pos), mean_neg = fp32(S_neg / c_neg) (0 for an
 * empty side).
 *   SGC_BIN_SBC: the side with the larger mean is sent (positive on a tie;
 *     nothing if the segment holds only zeros): out_idx gets that side's
 *     indices (ascending), out_counts the per-segment/total counts,
 *     out_means[t] the signed mean (+mean_pos or -mean_neg, 0 if empty).
 *     residual[i] <- fp32(v - mean) on the sent side, v for every other
 *     kept entry.  out_codes is ignored.
 *   SGC_BIN_2BIT: every kept entry gets code 1 (v > 0, value +mean_pos),
 *     2 (v < 0, value -mean_neg) or 0 (v = +-0, value +0): 2 bits per
 *     entry, LSB-first, 16 per uint32 of out_codes [ceil(total/16) words];
 *     out_means[2t] = +mean_pos, out_means[2t+1] = -mean_neg; out_counts =
 *     counts; out_idx (may be NULL) receives a copy of idx.
 *     residual[i] <- fp32(v - value).
 * residual [device, n] must hold +0 at the kept positions (as compress
 * leaves it), or -- with SGC_BIN_HELD or-ed into mode -- acc, that is val,
 * at the kept positions (as compress with SGC_HOLD_KEPT leaves it); the
 * result is the same, and only the entries whose value changes are written
 * (SBC: the sent side; 2-bit: codes 1 and 2).  Means match a sequential
 * double-precision sum within 1 ulp of fp32 (the summation order differs). */
size_t sgc_binarize_workspace(const sgc_layout* layout, int64_t cap);
int sgc_binarize(const sgc_layout* layout, int32_t mode,
                 const int32_t* idx, const float* val, const int64_t* counts, int64_t cap,
                 float* residual, int32_t* out_idx, int64_t* out_counts, float* out_means,
                 uint32_t* out_codes, void* ws, size_t ws_bytes, sgc_stream_t stream);

/* ------------------------------------------------------------------------
 * Rice-code the index gaps ([SBC] §II Optimal Position Encoding: distances
 * between nonzeros are Golomb coded; [SBC] appendix A: shapes are known).
 *
 * Streams: SGC_GLOBAL -> one stream of counts[nseg] global indices;
 * SGC_PER_SEGMENT -> stream t holds segment t's counts[t] indices relative
 * to the segment start.  Per stream the gap z = pos - prev - 1 (prev = -1
 * first) is coded as floor(z / 2^b) one-bits, a zero-bit, then the b low
 * bits of z least-significant first.  Stream bit i is bit (i mod 32) of its
 * word i / 32; each stream starts on a word boundary of out_words, pad bits
 * are 0.  out_word_off [device, nstreams+1] = first word of each stream and
 * the total; out_nbits [device, nstreams] = bits per stream;
 * out_chunk_off [device] = the chunk table, the decoder's entry points: for
 * codes 0, 256, 512, ... of stream 0, then of stream 1, ..., two uint64
 * entries each: the stream-relative bit offset of the code and the stream-
 * relative position reached before it (previous position + 1; 0 for the
 * stream's first code).  b in [0, 30].  word_cap / chunk_cap (uint64
 * entries) must be at least sgc_encode_word_bound / sgc_encode_chunk_bound
 * (else SGC_ENOSPC): those bounds hold for any counts with total <= cap.
 * Indices that are not strictly ascending inside a stream set
 * SGC_STATUS_BAD_INPUT.                                                     */
int64_t sgc_encode_word_bound(const sgc_layout* layout, int32_t scope, int32_t b, int64_t cap);
int64_t sgc_encode_chunk_bound(const sgc_layout* layout, int32_t scope, int64_t cap);
size_t sgc_encode_workspace(const sgc_layout* layout, int32_t scope, int64_t cap);
int sgc_encode(const sgc_layout* layout, int32_t scope, int32_t b,
               const int32_t* idx, const int64_t* counts, int64_t cap,
               uint32_t* out_words, int64_t word_cap, uint64_t* out_word_off,
               uint64_t* out_nbits, uint64_t* out_chunk_off, int64_t chunk_cap,
               uint32_t* dstatus, void* ws, size_t ws_bytes, sgc_stream_t stream);

/* ------------------------------------------------------------------------
 * Decode W messages and add them into a dense buffer ([SBC] §I: updates
 * are combined by a server or an all-reduce; [AHB19] Abstract: the global
 * sparse update is combined with the local dense gradient; [SBC] appendix
 * A: decoding uses the known shapes).
 *
 *   out = 0 | base | out (init); then for w = 0 .. W-1 in order, for every
 *   entry present in message w: out[pos] <- fp32(out[pos] + value).
 * Values: RAW_F32 / GOLOMB_F32 -> val[j]; GOLOMB_SBC -> means[t] of the
 * entry's segment; *_2BIT -> code 0 -> +0, 1 -> means[2t], 2 -> means[2t+1].
 * The segment of entry j follows from counts (entries are ascending).  A
 * message whose stream overruns its bits, leaves bits unread, disagrees
 * with either entry of its chunk table, holds a position >= its stream's
 * size, has raw indices that are not strictly ascending or in [0, n), or a
 * 2-bit code 3, is skipped entirely and sets SGC_STATUS_CORRUPT.
 * msgs [host, W descriptors of device pointers].  base [device, n] is read
 * for SGC_INIT_BASE only.  out [device, n].                                */
typedef struct {
    int32_t format;            /* SGC_MSG_* */
    int32_t scope;             /* GOLOMB formats: stream layout, as given to sgc_encode */
    int32_t rice_b;            /* GOLOMB formats: the b given to sgc_encode */
    int32_t reserved;          /* 0 */
    int64_t cap;               /* [host] upper bound on counts[nseg] */
    const int64_t* counts;     /* [nseg+1] entries per segment, then the total */
    const int32_t* idx;        /* RAW_*: global indices, ascending */
    const float* val;          /* RAW_F32, GOLOMB_F32: one value per entry */
    const uint32_t* codes;     /* *_2BIT: 2-bit codes, 16 per word */
    const float* means;        /* GOLOMB_SBC: [nseg]; *_2BIT: [2*nseg] */
    const uint32_t* words;     /* GOLOMB_*: the coded streams */
    const uint64_t* word_off;  /* GOLOMB_*: [nstreams+1] */
    const uint64_t* nbits;     /* GOLOMB_*: [nstreams] */
    const uint64_t* chunk_off; /* GOLOMB_*: chunk table (bit offset, position reached) pairs */
} sgc_message;

size_t sgc_decode_accumulate_workspace(const sgc_layout* layout, const sgc_message* msgs, int32_t W);
int sgc_decode_accumulate(const sgc_layout* layout, const sgc_message* msgs, int32_t W,
                          int32_t init, const float* base, float* out,
                          uint32_t* dstatus, void* ws, size_t ws_bytes, sgc_stream_t stream);

/* ------------------------------------------------------------------------
 * Measurement hook (benchmarks only).  While set, every sgc_compress call
 * (modes SGC_EXACT and SGC_SAMPLED) records `start` on its stream just
 * before launching the fused residual-add + candidate pass and `stop` just
 * after it, so the caller can time that one kernel with its own events.
 * start / stop are hipEvent_t handles owned by the caller; NULL, NULL
 * clears the hook.  Process-wide and not thread-safe: for single-threaded
 * measurement only.  Returns SGC_EINVAL if exactly one handle is NULL.    */
int sgc_set_pass_events(void* start, void* stop);

#ifdef __cplusplus
}
#endif

#endif /* SGC_H */
