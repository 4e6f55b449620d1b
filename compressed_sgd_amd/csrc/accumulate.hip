// accumulate.hip -- decode W messages and add them into a dense buffer
// (sgc_decode_accumulate).
//
// [SBC] §I: the clients' updates are combined by a central server or an
// all-reduce; [AHB19] Abstract: the compressed global update is combined
// with the node's own uncompressed local gradient (SGC_INIT_BASE);
// [SBC] appendix A: decoding uses the tensor shapes both ends know.
//
// GPU design, per batch of messages (blockIdx.y = message):
//  setup   validate counts / stream tables, entry and chunk prefixes;
//  raw     check that raw positions ascend; resolve 2-bit values;
//  decode  Rice streams: one thread per 256-code chunk starts from its
//          chunk-table entry (bit offset, position reached), decodes from
//          a copy of its words in LDS, writes positions (and resolved SBC
//          / 2-bit values), and checks that it ends exactly where the next
//          chunk's entry says (or at the stream's bit count);
//  fill    the output-tile table from the marks the two passes above left.
// Every message then has a sorted list of 16-bit positions (each less its
// output tile's first element), a value list (its own val if fp32) and,
// per output tile, the index of its first entry at or beyond the tile.
// The merge then gives
// each output tile to one workgroup: the initial tile and every message's
// entries for it are loaded in parallel, each thread applies the messages
// in order to the elements it owns (no atomics), and the tile is stored
// once: the dense output is written exactly once, in a fixed order.
#include "sgc_common.h"

#include <type_traits>

namespace sgc {

typedef float f4a __attribute__((ext_vector_type(4)));
typedef int32_t i4v __attribute__((ext_vector_type(4)));

constexpr int kBatch = 16;    // messages per decode launch
constexpr int kMerge = 16;    // messages per merge launch
constexpr int kFillPer = 16;  // output tiles per thread in the tile-table fill
constexpr int64_t kFillTiles = (int64_t)kBlock * kFillPer;

struct MsgWs {
    int64_t* estart;  // [nseg+1] entry prefix per segment
    int64_t* scnt;    // [S] codes per stream
    int64_t* sent;    // [S+1] first entry per stream
    int64_t* sbase;   // [S] first element of each stream
    int64_t* ssize;   // [S]
    int64_t* chpre;   // [S+1] chunk prefix
    uint16_t* pos;    // [cap] decoded positions less their output tile's first element
    int32_t* bmax;    // [cdiv(ntiles, kFillTiles)] largest tile mark of each block (fill)
    float* val;       // [cap] resolved values
    int32_t* tstart;  // [ntiles+1] first entry at or beyond each output tile
    uint32_t* bad;    // [1]
    int64_t* total;   // [1]
};

struct MsgIn {
    int32_t format, scope, b, S;
    int64_t cap, wbound;
    const int64_t* counts;
    const int32_t* idx;
    const float* val;
    const uint32_t* codes;
    const float* means;
    const uint32_t* words;
    const uint64_t* word_off;
    const uint64_t* nbits;
    const uint64_t* chunk_off;
};

struct Batch {
    int32_t n;
    MsgIn in[kBatch];
    MsgWs ws[kBatch];
};

struct MergeBatch {
    int32_t n;
    const uint16_t* pos[kMerge];  // entry positions less their output tile's first element
    const float* val[kMerge];
    const int32_t* tstart[kMerge];
    const uint32_t* bad[kMerge];
};

static bool is_golomb(int32_t f) { return f == SGC_MSG_GOLOMB_F32 || f == SGC_MSG_GOLOMB_SBC || f == SGC_MSG_GOLOMB_2BIT; }
static bool is_2bit(int32_t f) { return f == SGC_MSG_RAW_2BIT || f == SGC_MSG_GOLOMB_2BIT; }

static int32_t msg_streams(const sgc_layout* L, const sgc_message& m)
{
    return is_golomb(m.format) ? (m.scope == SGC_GLOBAL ? 1 : L->nseg) : 1;
}

static int64_t msg_nch(const sgc_layout* L, const sgc_message& m)
{
    return cdiv(m.cap, (int64_t)SGC_CHUNK_CODES) + msg_streams(L, m) + 1;
}

static int64_t out_tiles(const sgc_layout* L) { return cdiv(L->n, kOutTile); }

static void carve_msg(Carver& c, const sgc_layout* L, const sgc_message& m, MsgWs* w)
{
    const int64_t S = msg_streams(L, m), nch = msg_nch(L, m);
    w->estart = c.take<int64_t>(L->nseg + 1);
    w->scnt = c.take<int64_t>(S);
    w->sent = c.take<int64_t>(S + 1);
    w->sbase = c.take<int64_t>(S);
    w->ssize = c.take<int64_t>(S);
    w->chpre = c.take<int64_t>(S + 1);
    w->pos = c.take<uint16_t>(m.cap);
    w->val = c.take<float>(m.cap);
    w->tstart = c.take<int32_t>(out_tiles(L) + 1);
    w->bmax = c.take<int32_t>(cdiv(out_tiles(L), kFillTiles));
    w->bad = c.take<uint32_t>(1);
    w->total = c.take<int64_t>(1);
}

// ------------------------------------------------------------------ setup
// Every thread clears the output-tile marks (-1: no mark); workgroup 0 of each message checks its
// tables, one thread per segment / stream in rounds (workgroup scans for the
// prefixes, an OR over the workgroup for the verdict).  A message that fails
// any check is skipped whole: its stream tables are cleared.
__global__ __launch_bounds__(kBlock) void k_msg_setup(Batch B, const int64_t* __restrict__ seg_off, int32_t nseg,
                                                     int64_t ntiles)
{
    const int m = blockIdx.y;
    const MsgIn& in = B.in[m];
    const MsgWs& w = B.ws[m];
    for (int64_t t = (int64_t)blockIdx.x * kBlock + threadIdx.x; t < ntiles; t += (int64_t)gridDim.x * kBlock)
        w.tstart[t] = -1;
    if (blockIdx.x) return;
    __shared__ int64_t tmp[kBlock / 64 + 1];
    const int64_t n = seg_off[nseg];
    bool bad = false;
    // entry prefix per segment; every count within [0, the room left below cap]
    int64_t e = 0;
    for (int64_t t0 = 0; t0 < nseg; t0 += kBlock) {
        const int64_t t = t0 + threadIdx.x;
        const bool on = t < nseg;
        const int64_t raw = on ? in.counts[t] : 0;
        const int64_t c = raw < 0 ? 0 : (raw > in.cap ? in.cap : raw);
        int64_t te;
        const int64_t xe = e + block_scan_excl<kBlock, int64_t>(c, tmp, &te);
        bad |= on && (raw < 0 || raw > in.cap - xe);
        if (on) w.estart[t] = xe;
        e += te;
    }
    bad = __syncthreads_or(bad);  // also makes every estart entry visible to the workgroup
    if (threadIdx.x == 0) w.estart[nseg] = e;
    if (bad || in.counts[nseg] != e) bad = true;
    const bool golomb = in.format >= SGC_MSG_GOLOMB_F32;
    const bool glob = !golomb || in.scope == SGC_GLOBAL;
    int64_t se = 0, ch = 0;
    if (!bad) {  // uniform
        for (int64_t s0 = 0; s0 < in.S; s0 += kBlock) {
            const int64_t s = s0 + threadIdx.x;
            const bool on = s < in.S;
            int64_t cnt = 0;
            bool sbad = false;
            if (on) {
                // the total e stands for estart[nseg] (thread 0 stores it, unsynchronised)
                cnt = glob ? e : (s + 1 == nseg ? e : w.estart[s + 1]) - w.estart[s];
                const int64_t size = glob ? n : seg_off[s + 1] - seg_off[s];
                w.scnt[s] = cnt;
                w.sbase[s] = glob ? 0 : seg_off[s];
                w.ssize[s] = size;
                sbad = cnt > size;
                if (golomb) {
                    const uint64_t w0 = in.word_off[s], w1 = in.word_off[s + 1];
                    // streams follow one another from word 0; each has the words its bits need
                    if ((s == 0 && w0 != 0) || w1 < w0 || (w1 - w0) != (in.nbits[s] + 31) / 32 ||
                        w1 > (uint64_t)in.wbound)
                        sbad = true;
                    if ((cnt > 0) != (in.nbits[s] > 0)) sbad = true;  // codes take at least one bit each
                }
            }
            int64_t tse, tch;
            const int64_t xse = se + block_scan_excl<kBlock, int64_t>(cnt, tmp, &tse);
            const int64_t xch =
                ch + block_scan_excl<kBlock, int64_t>(golomb ? cdiv(cnt, (int64_t)SGC_CHUNK_CODES) : 0, tmp, &tch);
            if (on) {
                w.sent[s] = xse;
                w.chpre[s] = xch;
            }
            bad |= sbad;
            se += tse;
            ch += tch;
        }
    }
    bad = __syncthreads_or(bad);
    if (bad) {
        for (int64_t s = threadIdx.x; s < in.S; s += kBlock) {
            w.scnt[s] = 0;
            w.sent[s] = 0;
            w.chpre[s] = 0;
        }
        se = 0;
        ch = 0;
    }
    if (threadIdx.x != 0) return;
    w.sent[in.S] = se;
    w.chpre[in.S] = ch;
    w.bad[0] = bad ? 1u : 0u;
    w.total[0] = bad ? 0 : e;
    w.tstart[ntiles] = (int32_t)(bad ? 0 : e);
}

// ---------------------------------------------------- entries, tile table
// After decoding, every message is a list of ascending positions, each
// stored less its output tile's first element in 16 bits.  The output-tile
// table holds, per tile, the first entry at or beyond the tile's first
// element.  It is built as marks and a prefix maximum: an entry j whose
// tile lies past the previous entry's marks the tile after the previous
// entry's (every tile from there up to j's own has j as its first entry),
// and a stream's last entry marks the tile after its own with the entry
// count so far (a lower bound when the next stream starts in the same tile;
// marks on one tile are kept by their maximum).  Marks grow with the tile
// (entries ascend), so each tile's value is the largest mark at or before
// it; tiles before any mark take 0.  Raw messages: one thread per entry
// checks the order (raw input is not trusted), stores the 16-bit position,
// resolves raw 2-bit values and writes its mark.  Coded messages: the
// decoder writes the marks as it goes.
constexpr int kEntPer = 8;  // entries per thread per round, loads all in flight

__global__ __launch_bounds__(kBlock) void k_msg_entries(Batch B, int32_t nseg, int64_t n, int64_t ntiles)
{
    const int m = blockIdx.y;
    const MsgIn& in = B.in[m];
    const MsgWs& w = B.ws[m];
    if (in.format >= SGC_MSG_GOLOMB_F32 || w.bad[0]) return;  // the decoder writes the marks of a coded message
    const int64_t total = w.total[0];
    const int32_t* pos = in.idx;
    bool bad = false;
    const int64_t step = (int64_t)gridDim.x * kBlock * kEntPer;
    for (int64_t j0 = (int64_t)blockIdx.x * kBlock * kEntPer + threadIdx.x; j0 < total; j0 += step) {
        // clamped, unconditional loads (a guarded load is waited for at once)
        int32_t pc[kEntPer], pp[kEntPer];
#pragma unroll
        for (int u = 0; u < kEntPer; ++u) {
            const int64_t j = min(j0 + u * kBlock, total - 1);
            pc[u] = pos[j];
            pp[u] = pos[j > 0 ? j - 1 : 0];
        }
#pragma unroll
        for (int u = 0; u < kEntPer; ++u) {
            const int64_t j = j0 + u * kBlock;
            if (j >= total) break;
            const int64_t p = pc[u];
            const int64_t prev = j == 0 ? -1 : (int64_t)pp[u];
            if (p < 0 || p >= n || p <= prev) {
                bad = true;
                continue;
            }
            if (in.format == SGC_MSG_RAW_2BIT) {  // other formats: the merge reads the values directly
                const uint32_t code = (in.codes[j >> 4] >> (2 * (j & 15))) & 3u;
                const int64_t t = find_bucket(w.estart, (int64_t)nseg + 1, j);
                if (code == 3u) bad = true;
                w.val[j] = code == 0u ? 0.0f : code == 1u ? in.means[2 * t] : in.means[2 * t + 1];
            }
            w.pos[j] = (uint16_t)(p & (kOutTile - 1));
            const int64_t t1 = p >> kOutTileLog, t0 = prev < 0 ? 0 : (prev >> kOutTileLog) + 1;
            if (t0 <= t1) w.tstart[t0] = (int32_t)j;
            if (j == total - 1 && t1 + 1 < ntiles) w.tstart[t1 + 1] = (int32_t)total;
        }
    }
    if (bad) atomicOr(w.bad, 1u);
}

// The prefix maximum over the marks, in blocks of kFillTiles tiles: the
// largest mark of each block first, then every block's running maximum
// from the blocks before it.

__global__ __launch_bounds__(kBlock) void k_fill_max(Batch B, int64_t ntiles)
{
    __shared__ int32_t red[kBlock / 64];
    const MsgWs& w = B.ws[blockIdx.y];
    if (w.bad[0]) return;
    const int64_t t0 = (int64_t)blockIdx.x * kFillTiles;
    int32_t mx = -1;
#pragma unroll
    for (int i = 0; i < kFillPer; ++i) {
        const int64_t t = t0 + i * kBlock + threadIdx.x;
        mx = max(mx, t < ntiles ? w.tstart[t] : -1);
    }
    for (int d = 32; d >= 1; d >>= 1) mx = max(mx, __shfl_xor(mx, d, 64));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int v = 1; v < kBlock / 64; ++v) mx = max(mx, red[v]);
        w.bmax[blockIdx.x] = mx;
    }
}

__global__ __launch_bounds__(kBlock) void k_fill(Batch B, int64_t ntiles)
{
    __shared__ int32_t wmax[kBlock / 64];
    const MsgWs& w = B.ws[blockIdx.y];
    if (w.bad[0]) return;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    // the blocks before this one (a few dozen at most)
    int32_t carry = -1;
    for (int64_t q = threadIdx.x; q < (int64_t)blockIdx.x; q += kBlock) carry = max(carry, w.bmax[q]);
    for (int d = 32; d >= 1; d >>= 1) carry = max(carry, __shfl_xor(carry, d, 64));
    if (lane == 0) wmax[wave] = carry;
    __syncthreads();
    carry = -1;
    for (int v = 0; v < kBlock / 64; ++v) carry = max(carry, wmax[v]);
    __syncthreads();  // wmax is rewritten below
    // this block: kFillPer consecutive tiles per thread
    const int64_t t0 = (int64_t)blockIdx.x * kFillTiles + (int64_t)threadIdx.x * kFillPer;
    const bool whole = t0 + kFillPer <= ntiles;  // 16-byte loads and stores (the table is 256-byte aligned)
    int32_t v[kFillPer];
    if (whole) {
#pragma unroll
        for (int i = 0; i < kFillPer; i += 4) {
            const i4v x = *(const i4v*)(w.tstart + t0 + i);
            v[i] = x[0];
            v[i + 1] = x[1];
            v[i + 2] = x[2];
            v[i + 3] = x[3];
        }
    } else {
#pragma unroll
        for (int i = 0; i < kFillPer; ++i) v[i] = t0 + i < ntiles ? w.tstart[t0 + i] : -1;
    }
    int32_t run = -1;
#pragma unroll
    for (int i = 0; i < kFillPer; ++i) {
        run = max(run, v[i]);
        v[i] = run;
    }
    // exclusive maximum of the threads before this one
    int32_t x = run;
    for (int d = 1; d < 64; d <<= 1) {
        const int32_t y = __shfl_up(x, d, 64);
        if (lane >= d) x = max(x, y);
    }
    if (lane == 63) wmax[wave] = x;
    __syncthreads();
    int32_t before = carry;
    for (int u = 0; u < wave; ++u) before = max(before, wmax[u]);
    const int32_t up = __shfl_up(x, 1, 64);
    if (lane > 0) before = max(before, up);
#pragma unroll
    for (int i = 0; i < kFillPer; ++i) v[i] = max(max(v[i], before), 0);
    if (whole) {
#pragma unroll
        for (int i = 0; i < kFillPer; i += 4) *(i4v*)(w.tstart + t0 + i) = i4v{v[i], v[i + 1], v[i + 2], v[i + 3]};
    } else {
#pragma unroll
        for (int i = 0; i < kFillPer; ++i)
            if (t0 + i < ntiles) w.tstart[t0 + i] = v[i];
    }
}

// --------------------------------------------------------- Rice decoding
struct ChunkAt {
    int64_t s, q0, nc;
};

__device__ inline ChunkAt chunk_at(const MsgWs& w, int32_t S, int64_t c)
{
    ChunkAt a;
    a.s = find_bucket(w.chpre, (int64_t)S + 1, c);
    a.q0 = (c - w.chpre[a.s]) * SGC_CHUNK_CODES;
    const int64_t left = w.scnt[a.s] - a.q0;
    a.nc = left < SGC_CHUNK_CODES ? left : SGC_CHUNK_CODES;
    return a;
}

// One thread per chunk, one wavefront per workgroup.  Each lane first copies
// its chunk's words into its own LDS column (independent loads, no
// barrier: no lane reads another lane's column), then decodes from LDS, so
// the decode loop issues no global loads at all and never waits on memory
// behind its own stores (one counter tracks both on this GPU).  A chunk
// whose words do not fit the column (very long gaps) reads global memory
// instead.  Bit positions are 32-bit, relative to the chunk's first word:
// a valid chunk spans less than 2^31 + 256 * 32 bits (its gaps sum to less
// than the stream's size), and a chunk-table entry that claims more is
// rejected.  Each code is read from a 32-bit window at its first bit; the
// unary run and the b low bits fit the window unless the gap is far above
// 2^b (then a loop reads further windows).
constexpr int kDecLanes = 64;
constexpr int kColWords = 120;  // LDS words per lane (the chunk's words plus slack), largest column
// Column sizes: a chunk of 256 Rice codes with parameter b takes about
// 256 * (b + 2) bits when b suits the density; the smallest column that
// holds that with slack is used, so that more waves fit in LDS (a chunk
// that does not fit reads global memory instead).
__host__ __device__ constexpr int col_words_for(int b) { return b <= 6 ? 80 : b <= 9 ? 104 : kColWords; }
constexpr int kColCodes = 17;   // 2-bit code words per lane (256 entries span at most 17)
constexpr uint32_t kMaxChunkBits = 0x80000000u + SGC_CHUNK_CODES * 32u;
constexpr int kCopy = 8;        // words per round of the column copy

// 32 stream bits starting at chunk-relative bit r, from the lane's LDS column.
struct LdsBits {
    const uint32_t* col;  // word i at col[i * kDecLanes]
    __device__ uint32_t win(uint32_t r) const
    {
        const uint32_t i = r >> 5;
        const uint32_t lo = col[i * kDecLanes], hi = col[(i + 1) * kDecLanes];
        return (uint32_t)((((uint64_t)hi << 32) | lo) >> (r & 31));
    }
};

// The same from global memory; words at or past nw read as 0.
struct GlobalBits {
    const uint32_t* w;
    uint64_t nw, bit0;  // chunk-relative bit 0 is stream bit bit0
    __device__ uint32_t win(uint32_t r) const
    {
        const uint64_t a = bit0 + r, i = a >> 5;
        const uint32_t lo = i < nw ? w[i] : 0u, hi = i + 1 < nw ? w[i + 1] : 0u;
        return (uint32_t)((((uint64_t)hi << 32) | lo) >> (a & 31));
    }
};

// What one lane needs to decode its chunk.
struct ChunkJob {
    uint32_t b, relend;     // Rice parameter; the chunk's end bit (relative)
    int32_t nc;             // codes in the chunk
    int32_t j0;             // message entry of its first code
    int32_t prev;           // stream position of the entry before it (-1 at the stream's start)
    int32_t size, base;     // stream size and its first element
    int32_t t, tend;        // value segment of entry j0 and where its entries end
    int32_t* tstart;        // output-tile table
};

template <int FMT>
__device__ inline void seg_means(const MsgIn& in, int32_t t, float* m0, float* m1)
{
    if (FMT == SGC_MSG_GOLOMB_SBC) *m0 = in.means[t];
    if (FMT == SGC_MSG_GOLOMB_2BIT) {
        *m0 = in.means[2 * t];
        *m1 = in.means[2 * t + 1];
    }
}

// Decode one chunk from src starting at relative bit rel; false if corrupt.
// Returns the end bit and the last position through *rel_out / *prev_out.
// Errors are collected in a flag rather than taken as branches; after one,
// decoding goes on over garbage with every read clamped inside the chunk's
// words, and the chunk is rejected at the end.  Per code only the position
// is checked (it guards the tile-table marks); a code that starts or ends
// past the chunk's end bit shows in the end bit, which the caller compares
// with the chunk table (bit positions only grow).  Groups of four codes run
// without per-code activity tests except the last, partial group of a
// stream.
template <int FMT, typename Src>
__device__ __forceinline__ bool decode_chunk(const Src& src, uint32_t rel, const ChunkJob& J, const MsgIn& in, const MsgWs& w,
                             const uint32_t* code_col, uint32_t* rel_out, int32_t* prev_out)
{
    const uint32_t b = J.b, mask = (1u << b) - 1u, last_rd = J.relend - 1;
    uint32_t prev = (uint32_t)J.prev;  // stream position of the previous entry; -1 wraps to all ones
    bool err = false;
    float m0 = 0.0f, m1 = 0.0f;
    int32_t t = J.t, tend = J.tend;
    if (FMT != SGC_MSG_GOLOMB_F32) seg_means<FMT>(in, t, &m0, &m1);
    const bool vec = (J.j0 & 7) == 0;  // 16-byte aligned stores of 8 positions
    // output tile of the previous entry (before a stream's first entry: of the
    // stream's origin minus one; arithmetic shift, so -1 stays -1)
    int32_t tp = (J.base + (int32_t)prev) >> kOutTileLog;
    // positions of codes i0 .. i0+3 to pb (stored by the caller), one code at
    // a time with every check in place: partial groups, and whole groups
    // that hold a long code
    auto careful = [&](int32_t i0, auto full, int32_t (&pb)[4]) __attribute__((always_inline)) {
        constexpr bool kFull = decltype(full)::value;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const bool act = kFull || i0 + q < J.nc;
            const uint32_t win = src.win(min(rel, last_rd));
            const uint32_t ones = __builtin_ctzg(~win, 32);
            uint32_t len = ones + 1 + b;
            uint32_t z = (ones << b) | ((win >> min(ones, 31u) >> 1) & mask);
            if (__builtin_expect(len > 32, 0)) {  // the unary run and the low bits leave the window: read on
                uint64_t qq = 0;
                uint32_t r = rel;
                bool fin = false;
                while (!fin && r < J.relend) {
                    const uint32_t o = __builtin_ctzg(~src.win(r), 32);
                    qq += o;
                    r += o < 32 ? o + 1 : 32;
                    fin = o < 32;
                }
                uint32_t rem = 0;
                if (b) rem = src.win(min(r, last_rd)) & mask;
                const uint64_t zz = (qq << b) | rem;
                err |= act && (!fin || qq >> 31 || zz >= (uint64_t)J.size);
                z = (uint32_t)zz;
                len = r + b - rel;
            }
            const uint32_t pu = prev + 1 + z;  // below 2^32 unless already in error
            err |= act && pu >= (uint32_t)J.size;
            // output-tile table: an entry in a later tile than the entry before
            // it marks the tile after that entry's.  Global positions are below
            // 2^31.  A corrupt chunk may mark wrongly: its message is dropped
            // whole.
            const int32_t t1 = (int32_t)(J.base + pu) >> kOutTileLog;
            if (__builtin_expect(act && !err && t1 != tp, 0)) J.tstart[tp + 1] = J.j0 + i0 + q;
            if (act) {
                rel += len;
                prev = pu;
                tp = t1;
            }
            pb[q] = (int32_t)((uint32_t)J.base + prev);
        }
    };
    // a whole group without a branch per code (long codes and tile-table
    // marks are rare): the four codes first, then one wave vote for a long
    // code among them (such a lane redoes its group carefully, from the
    // state before it) and one for marks to write
    auto fast = [&](int32_t i0, int32_t (&pb)[4]) __attribute__((always_inline)) {
        const uint32_t rel0 = rel, prev0 = prev;
        const int32_t tp0 = tp;
        const bool err0 = err;
        bool slow = false;
        uint32_t marks = 0, top = 0;
        int32_t tps[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t win = src.win(min(rel, last_rd));
            const uint32_t ones = __builtin_ctzg(~win, 32);
            const uint32_t run = ones + 1;  // the unary run and its stop bit
            const uint32_t len = run + b;
            // the low bits follow the stop bit; run & 31 is the shift the
            // hardware takes anyway, and only ever differs from run for a
            // 32-bit run: then b = 0 and there are no low bits, or the code
            // is long and the group is redone carefully
            const uint32_t z = (ones << b) | ((win >> (run & 31u)) & mask);
            slow |= len > 32;
            const uint32_t pu = prev + 1 + z;
            top = max(top, pu);
            const int32_t t1 = (int32_t)(J.base + pu) >> kOutTileLog;
            marks |= t1 != tp ? 1u << q : 0u;
            tps[q] = tp;
            rel += len;
            prev = pu;
            tp = t1;
            pb[q] = (int32_t)((uint32_t)J.base + prev);
        }
        // One check for the group: with codes of at most 32 bits each gap is
        // below 2^31, so the first position at or past the stream's size is
        // formed without wrapping (every one before it is below the size) and
        // the largest of the four is at or past it too.  A corrupt chunk
        // writes no marks (its message is dropped whole).
        err |= top >= (uint32_t)J.size;
        if (err) marks = 0;
        if (__builtin_expect(__any(slow), 0)) {
            if (slow) {
                rel = rel0;
                prev = prev0;
                tp = tp0;
                err = err0;
                marks = 0;  // the careful pass writes its own
                careful(i0, std::true_type{}, pb);
            }
        }
        if (__builtin_expect(__any(marks != 0u), 0)) {
            // the first crossing of the group: every code before it lies in
            // the tile the group started in, so its mark goes to the tile
            // after that one -- a single store
            if (marks != 0u) J.tstart[tp0 + 1] = J.j0 + i0 + __builtin_ctz(marks);
            marks &= marks - 1u;
            if (__builtin_expect(__any(marks != 0u), 0)) {  // more than one tile crossed in four codes
#pragma unroll
                for (int q = 1; q < 4; ++q)
                    if ((marks >> q) & 1u) J.tstart[tps[q] + 1] = J.j0 + i0 + q;
            }
        }
    };
    // codes i0 .. i0+3: positions to pb (stored by the caller), then the
    // values (SBC and 2-bit formats), stored here
    auto group = [&](int32_t i0, auto full, int32_t (&pb)[4]) __attribute__((always_inline)) {
        constexpr bool kFull = decltype(full)::value;
        if constexpr (kFull) fast(i0, pb);
        else careful(i0, full, pb);
        if constexpr (FMT != SGC_MSG_GOLOMB_F32) {
            float vb[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                vb[q] = 0.0f;
                if (kFull || i0 + q < J.nc) {
                    const int32_t j = J.j0 + i0 + q;
                    while (j >= tend) {  // entered the next segment (global scope): rare
                        ++t;
                        tend = (int32_t)w.estart[t + 1];
                        seg_means<FMT>(in, t, &m0, &m1);
                    }
                    if (FMT == SGC_MSG_GOLOMB_SBC) {
                        vb[q] = m0;
                    } else {
                        const int32_t r = i0 + q + (J.j0 & 15);  // entry within the lane's code words
                        const uint32_t code = (code_col[(r >> 4) * kDecLanes] >> (2 * (r & 15))) & 3u;
                        err |= code == 3u;
                        vb[q] = code == 0u ? 0.0f : code == 1u ? m0 : m1;
                    }
                }
            }
            const int32_t jb = J.j0 + i0;
            if (kFull && vec) {
                *(f4a*)(w.val + jb) = f4a{vb[0], vb[1], vb[2], vb[3]};
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    if (kFull || i0 + q < J.nc) w.val[jb + q] = vb[q];
            }
        }
    };
    // positions are stored less their output tile's first element, in 16
    // bits (the merge knows each entry's tile from the tile table)
    constexpr int32_t kOff = (int32_t)kOutTile - 1;
    auto pair = [](int32_t a, int32_t b) -> int32_t { return (a & kOff) | ((b & kOff) << 16); };
    auto store4 = [&](int32_t i0, const int32_t (&pb)[4], auto full) __attribute__((always_inline)) {
        constexpr bool kFull = decltype(full)::value;
        const int32_t jb = J.j0 + i0;
        if (kFull && vec) {
            *(int2*)(w.pos + jb) = int2{pair(pb[0], pb[1]), pair(pb[2], pb[3])};
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (kFull || i0 + q < J.nc) w.pos[jb + q] = (uint16_t)(pb[q] & kOff);
        }
    };
    int32_t i0 = 0;
    int32_t pb[4];
    // whole blocks of 64 codes: the positions stay in registers and leave as
    // eight back-to-back 16-byte stores, one whole 128-byte cache line (every
    // lane writes its own chunk, so stores in 16-byte pieces left partly
    // written lines: 2.4 times the position bytes reached memory)
    if (vec) {
        for (; i0 + 64 <= J.nc; i0 += 64) {
            i4v buf[8];
#pragma unroll
            for (int g = 0; g < 8; ++g) {
                group(i0 + 8 * g, std::true_type{}, pb);
                const int32_t lo0 = pair(pb[0], pb[1]), lo1 = pair(pb[2], pb[3]);
                group(i0 + 8 * g + 4, std::true_type{}, pb);
                buf[g] = i4v{lo0, lo1, pair(pb[0], pb[1]), pair(pb[2], pb[3])};
            }
#pragma unroll
            for (int g = 0; g < 8; ++g) *(i4v*)(w.pos + J.j0 + i0 + 8 * g) = buf[g];
        }
    }
    for (; i0 + 4 <= J.nc; i0 += 4) {
        group(i0, std::true_type{}, pb);
        store4(i0, pb, std::true_type{});
    }
    if (i0 < J.nc) {
        group(i0, std::false_type{}, pb);
        store4(i0, pb, std::false_type{});
    }
    *rel_out = rel;
    *prev_out = (int32_t)prev;
    return !err;
}

template <int FMT, int COLW>
__device__ __forceinline__ void decode_lanes(const MsgIn& in, const MsgWs& w, int32_t nseg, int64_t ntiles, uint32_t* col,
                                             uint32_t* ccol)
{
    const int lane = threadIdx.x;
    const int64_t nch = w.chpre[in.S];
    bool bad = false;
    for (int64_t c = (int64_t)blockIdx.x * kDecLanes + lane; c < nch; c += (int64_t)gridDim.x * kDecLanes) {
        const ChunkAt a = chunk_at(w, in.S, c);
        const uint64_t bit0 = in.chunk_off[2 * c], reached = in.chunk_off[2 * c + 1];
        const bool last = c + 1 >= w.chpre[a.s + 1];
        const uint64_t nbits = in.nbits[a.s];
        const uint64_t bit1 = last ? nbits : in.chunk_off[2 * (c + 1)];
        const int64_t size = w.ssize[a.s];
        if ((a.q0 == 0 && (bit0 != 0 || reached != 0)) || reached > (uint64_t)size || bit1 <= bit0 ||
            bit1 > nbits || bit1 - bit0 > kMaxChunkBits) {
            bad = true;
            continue;
        }
        const uint32_t* words = in.words + in.word_off[a.s];
        const uint64_t nw = in.word_off[a.s + 1] - in.word_off[a.s];
        ChunkJob J;
        J.b = (uint32_t)in.b;
        J.nc = (int32_t)a.nc;
        J.j0 = (int32_t)(w.sent[a.s] + a.q0);
        J.prev = (int32_t)reached - 1;
        J.size = (int32_t)size;
        J.base = (int32_t)w.sbase[a.s];
        J.t = 0;
        J.tend = INT32_MAX;
        J.tstart = w.tstart;
        if (FMT != SGC_MSG_GOLOMB_F32) {
            J.t = (int32_t)(in.scope == SGC_PER_SEGMENT ? a.s : find_bucket(w.estart, (int64_t)nseg + 1, (int64_t)J.j0));
            J.tend = in.scope == SGC_PER_SEGMENT ? INT32_MAX : (int32_t)w.estart[J.t + 1];
        }
        const uint32_t* code_col = nullptr;
        if (FMT == SGC_MSG_GOLOMB_2BIT) {  // the chunk's 2-bit code words
            const int32_t cw0 = J.j0 >> 4, ncw = ((J.j0 + J.nc - 1) >> 4) - cw0 + 1;
            for (int32_t i = 0; i < ncw; ++i) ccol[i * kDecLanes + lane] = in.codes[cw0 + i];
            code_col = ccol + lane;
        }
        // words [bit0/32, bit1/32 + 1]: every window read before bit1 lies inside
        const uint64_t wlo = bit0 >> 5;
        const uint64_t need = (bit1 >> 5) + 2 - wlo;
        uint32_t rel_end;
        int32_t prev_end;
        bool ok;
        J.relend = (uint32_t)(bit1 - (wlo << 5));
        if (need <= (uint64_t)COLW) {
            // kCopy loads at a time, clamped into the stream and all in flight;
            // words past the stream's end read as 0 (a valid chunk has
            // nw >= 1 and wlo < nw)
            const uint32_t nd = (uint32_t)need;
            for (uint32_t i0 = 0; i0 < nd; i0 += kCopy) {
                uint32_t v[kCopy];
#pragma unroll
                for (int q = 0; q < kCopy; ++q) v[q] = words[min(wlo + i0 + q, nw - 1)];
#pragma unroll
                for (int q = 0; q < kCopy; ++q)
                    if (i0 + q < nd) col[(i0 + q) * kDecLanes + lane] = wlo + i0 + q < nw ? v[q] : 0u;
            }
            ok = decode_chunk<FMT>(LdsBits{col + lane}, (uint32_t)(bit0 & 31), J, in, w, code_col, &rel_end, &prev_end);
        } else {
            ok = decode_chunk<FMT>(GlobalBits{words, nw, wlo << 5}, (uint32_t)(bit0 & 31), J, in, w, code_col,
                                   &rel_end, &prev_end);
        }
        if (!ok) {
            bad = true;
            continue;
        }
        if (!last) {
            // the next chunk must start exactly where this one ended
            if (rel_end != J.relend || in.chunk_off[2 * (c + 1) + 1] != (uint64_t)(prev_end + 1)) bad = true;
        } else if (rel_end != J.relend) {
            bad = true;  // bits left over
        } else if (J.nc > 0) {
            // the stream's last entry marks the tile after its own with the
            // entry count so far.  A later stream may still have entries in
            // that entry's tile, so this count is only a lower bound, and
            // other streams may mark the same tile: the largest mark is right.
            const int64_t te = (((int64_t)J.base + prev_end) >> kOutTileLog) + 1;
            if (te < ntiles) atomicMax(w.tstart + te, J.j0 + J.nc);
        }
    }
    if (bad) atomicOr(w.bad, 1u);
}

// COLW: column words per lane; CODES: the batch holds 2-bit messages (their
// code words get a column of their own).  LDS per workgroup is what limits
// how many decoding waves a CU holds.
template <int COLW, bool CODES>
__global__ __launch_bounds__(kDecLanes) void k_msg_decode(Batch B, int32_t nseg, int64_t ntiles)
{
    __shared__ uint32_t col[COLW * kDecLanes];
    __shared__ uint32_t ccol[(CODES ? kColCodes : 1) * kDecLanes];
    const int m = blockIdx.y;
    const MsgIn& in = B.in[m];
    const MsgWs& w = B.ws[m];
    if (w.bad[0]) return;
    switch (in.format) {
    case SGC_MSG_GOLOMB_F32: decode_lanes<SGC_MSG_GOLOMB_F32, COLW>(in, w, nseg, ntiles, col, ccol); break;
    case SGC_MSG_GOLOMB_SBC: decode_lanes<SGC_MSG_GOLOMB_SBC, COLW>(in, w, nseg, ntiles, col, ccol); break;
    case SGC_MSG_GOLOMB_2BIT:
        if constexpr (CODES) decode_lanes<SGC_MSG_GOLOMB_2BIT, COLW>(in, w, nseg, ntiles, col, ccol);
        break;
    default: break;
    }
}

template <bool CODES>
static void launch_decode(int colw, dim3 grid, const Batch& B, int32_t nseg, int64_t ntiles, hipStream_t s)
{
    if (colw == col_words_for(6)) k_msg_decode<col_words_for(6), CODES><<<grid, kDecLanes, 0, s>>>(B, nseg, ntiles);
    else if (colw == col_words_for(9))
        k_msg_decode<col_words_for(9), CODES><<<grid, kDecLanes, 0, s>>>(B, nseg, ntiles);
    else k_msg_decode<kColWords, CODES><<<grid, kDecLanes, 0, s>>>(B, nseg, ntiles);
}

// ------------------------------------------------------------------ merge
// Persistent workgroups over the output tiles (kOutTile elements each), in
// runs of kTileRun consecutive tiles: workgroup i takes runs i, i + G, i + 2G,
// ... for a grid of G.  Spread out like this, clustered entries (runs of
// dense tiles, as the rows of a Zipf-sampled embedding give) load every
// workgroup instead of the few that a contiguous range would give them to;
// in runs, the cache line that holds the end of one tile's entries and the
// start of the next is fetched once rather than by two workgroups (single
// tiles: 1.44 times the entry bytes were fetched).  A group of threads per message (a power of two)
// follows that message's entries, which stay in the registers of the thread
// that loaded them.  Per tile:
//  1  the tile's initial contents go to LDS; every entry marks its message
//     in the 16-bit message mask of its tile position (LDS atomic or: the
//     mask does not depend on the order);
//  2  each entry reads its position's mask: its rank there is the number of
//     lower messages present.  Rank-0 entries add their value in place (no
//     other thread touches that element in this step);
//  3  where messages meet, rank 1, 2, ... follow, one step each, with a
//     barrier between steps (usually none is needed);
// and the tile is stored once (coalesced).  Every element receives its
// values in message order, so the result does not depend on scheduling.
// One mask serves every tile: it is cleared after its last read, and a
// barrier separates that clear from the next tile's marks.
//
// Tiles are 8192 elements: the fixed cost per tile (its barriers and
// bookkeeping) is what bounds the merge at low densities, and halving the
// tile count took 16 x 0.1% onto zeros from 1.09 to 0.93 ms.  kPre = 8 holds
// a message's share of a tile at 1% (82 entries on average) in 16 threads.
// The output and the initial contents are streamed with non-temporal
// stores and loads (each is touched once; 3-5% faster than plain ones).
// The kernel is built with and without initial contents to load: without
// them (sums onto zeros) it needs no registers for them and runs three
// workgroups per CU (the LDS limit); with them, two.  Each comes in two
// workgroup sizes (below).
//
// Software pipeline: while tile j of the sequence is worked on, the entries
// and initial contents of tile j+1 (LOAD only; and the entry-range bounds of
// tile j+2) are already in flight in registers.  In each iteration the stores of the previous tile are
// issued before the next loads: loads and stores share one completion
// counter here, so a wait for loads also waits for earlier stores, and
// those are then long done.  A tile whose entries do not fit the prefetch (a
// message with more than kPre * group-size entries in it, or more than
// kRound in all) is applied from memory instead, in rounds of kRound entries
// taken in message order.
constexpr int kTileRun = 4;  // consecutive tiles a workgroup takes in a row
constexpr int kPre = 8;      // entries per thread per tile (or round)
static_assert(kMerge <= 16, "message masks are 16 bits");
// The merge runs with NT threads per workgroup: 256, or 512 for sparse
// batches (few entries per tile: more waves per CU keep the output stream
// busy, 16 x 0.1% onto zeros 0.96 -> 0.86 ms; at 16 x 1% 512 threads were
// slower, 1.55 -> 1.69 ms).
constexpr int kMergeSparseEntries = 256;  // entries per tile (by capacity) up to which the batch is sparse
template <int NT>
struct MergeShape {
    static constexpr int kRound = kPre * NT;                    // entries per round
    static constexpr int kQ = (int)(kOutTile / (4 * NT));       // 16-byte words per thread in a tile
    static constexpr int kMaskWords = (int)(kOutTile / 2) / NT;  // mask words each thread clears
    static_assert(kMaskWords % 4 == 0, "mask clear in 16-byte words");
    static_assert((int64_t)kQ * 4 * NT == kOutTile, "a tile is whole 16-byte words per thread");
};

struct MergeLds {
    float tile[kOutTile];
    uint32_t mask[kOutTile / 2];  // 16-bit message mask per position, two per word
    int32_t a[2][kMerge], cnt[2][kMerge];
    int32_t total[3], fits[3], maxc[3];  // per tile, by tile index mod 3
};

// Wave 0: bookkeeping of the tile with range parity par and slot z: entry
// total, whether the prefetch holds all its entries, collision depth 1.
template <int NT>
__device__ inline void tile_meta(MergeLds& S, int par, int z, int32_t nmsg, int32_t cap_per_msg)
{
    const int lane = threadIdx.x;
    const int32_t c = lane < nmsg ? S.cnt[par][lane] : 0;
    int32_t total = c;
    for (int d = 32; d >= 1; d >>= 1) total += __shfl_xor(total, d, 64);
    const bool over = __any(c > cap_per_msg);
    if (lane == 0) {
        S.total[z] = total;
        S.fits[z] = !over && total <= MergeShape<NT>::kRound;
        S.maxc[z] = 1;
    }
}

template <int NT>
__device__ inline void clear_mask(uint32_t* mask)
{
    constexpr int MW = MergeShape<NT>::kMaskWords;
#pragma unroll
    for (int q = 0; q < MW / 4; ++q) *(i4v*)&mask[MW * threadIdx.x + 4 * q] = i4v{0, 0, 0, 0};
}

// Step 1: every entry (message k[i], tile position p[i] >= 0) marks its message.
__device__ inline void mark_entries(uint32_t* mask, const int32_t (&k)[kPre], const int32_t (&p)[kPre])
{
#pragma unroll
    for (int i = 0; i < kPre; ++i)
        if (p[i] >= 0) atomicOr(&mask[p[i] >> 1], (1u << k[i]) << (16 * (p[i] & 1)));
}

// Steps 2 and 3, after a barrier that follows the marks.  The mask is
// cleared after the barrier that ends its reads; the function ends with a
// barrier after both the last addition and the clear.
template <int NT>
__device__ inline void add_entries(MergeLds& S, uint32_t* mask, int z, const int32_t (&k)[kPre],
                                   const int32_t (&p)[kPre], const float (&v)[kPre])
{
    int32_t rk[kPre];
    int32_t deep = 1;
#pragma unroll
    for (int i = 0; i < kPre; ++i) {
        rk[i] = -1;
        if (p[i] < 0) continue;
        const uint32_t m = (mask[p[i] >> 1] >> (16 * (p[i] & 1))) & 0xffffu;
        rk[i] = __builtin_popcount(m & ((1u << k[i]) - 1u));
        deep = max(deep, __builtin_popcount(m));
        if (rk[i] == 0) S.tile[p[i]] = S.tile[p[i]] + v[i];
    }
    if (deep > 1) atomicMax(&S.maxc[z], deep);
    __syncthreads();
    clear_mask<NT>(mask);  // every read of the mask is done
    const int32_t depth = S.maxc[z];  // uniform
    if (depth == 1) __syncthreads();  // the clear ends before the next marks
    for (int32_t r = 1; r < depth; ++r) {
#pragma unroll
        for (int i = 0; i < kPre; ++i)
            if (rk[i] == r) S.tile[p[i]] = S.tile[p[i]] + v[i];
        __syncthreads();
    }
}

// Read by merge lanes that have no message, so that every tile-table load
// is unconditional.
__device__ int32_t g_zero_word = 0;

template <bool LOAD, int NT>
__global__ __launch_bounds__(NT) void k_merge(MergeBatch M, int32_t lg_tpm, int32_t init,
                                                 const float* __restrict__ base, float* __restrict__ out, int64_t n,
                                                 int64_t ntiles, uint32_t* status)
{
    __shared__ __align__(16) MergeLds S;
    const int tid = threadIdx.x;
    const int tpm = 1 << lg_tpm;  // threads per message slot
    const int mk = tid >> lg_tpm, ml = tid & (tpm - 1);
    const bool live = mk < M.n && !*M.bad[mk];
    // the batch's corrupt messages (their flags are final before the merge)
    // reach the caller's status word, from workgroup 0
    if (status && blockIdx.x == 0 && tid < 64) {
        const bool bad = tid < M.n && *M.bad[tid] != 0u;
        if (__ballot(bad) != 0ull && tid == 0) *status |= SGC_STATUS_CORRUPT;
    }
    const uint16_t* posk = live ? M.pos[mk] : nullptr;
    const float* valk = live ? M.val[mk] : nullptr;
    const int32_t* tsk = live ? M.tstart[mk] : nullptr;
    const float* src = init == SGC_INIT_BASE ? base : out;
    // this workgroup's tiles: the groups of kTileRun consecutive tiles numbered
    // blockIdx.x, + gridDim.x, + 2 gridDim.x, ... (j-th tile: tile(j); past
    // the sequence's end tile(j) >= ntiles)
    const int64_t ngr = (ntiles + kTileRun - 1) / kTileRun;
    if ((int64_t)blockIdx.x >= ngr) return;
    const int64_t G = gridDim.x;
    const int64_t my_groups = (ngr - (int64_t)blockIdx.x + G - 1) / G;
    const int64_t last_group = (int64_t)blockIdx.x + (my_groups - 1) * G;
    const int64_t J = (my_groups - 1) * kTileRun + min((int64_t)kTileRun, ntiles - last_group * kTileRun);
    auto tile = [&](int64_t j) -> int64_t {
        return ((int64_t)blockIdx.x + (j / kTileRun) * G) * kTileRun + (j % kTileRun);
    };

    // pipeline registers: the next tile's entries (positions in the tile, -1 for none) and initial contents
    int32_t n_pos[kPre];
    float n_val[kPre];
    constexpr int kQ = MergeShape<NT>::kQ;
    constexpr int kRound = MergeShape<NT>::kRound;
    f4a ini[kQ];
    // entry-range bounds, clamped to the message's entries (memory safety
    // does not depend on the tile table being right).  The table load is
    // unconditional (a lane without a message reads a zero word) and the
    // clamp is applied where the bound is used: a guarded load would be
    // waited for at once, together with every store issued before it.
    const int32_t* tsl = live ? tsk : &g_zero_word;
    auto ts_load = [&](int64_t t) -> int32_t { return tsl[live ? min(t, ntiles) : 0]; };
    const int32_t tot = live ? ts_load(ntiles) : 0;
    auto ts_fix = [&](int64_t t, int32_t raw) -> int32_t { return (live && t <= ntiles) ? min(max(raw, 0), tot) : 0; };
    auto ts = [&](int64_t t) -> int32_t { return ts_fix(t, ts_load(t)); };
    auto span = [](int32_t a, int32_t e) -> int32_t { return max(e - a, 0); };
    auto load_tile = [&](int64_t t, int32_t a, int32_t c) {
        const int64_t lo = t * kOutTile;
        const int32_t cnt = (int32_t)min((int64_t)kOutTile, n - lo);
#pragma unroll
        for (int i = 0; i < kPre; ++i) {
            const int32_t r = ml + i * tpm;
            n_pos[i] = -1;
            n_val[i] = 0.0f;
            if (r < c) {
                n_pos[i] = posk[a + r];
                n_val[i] = valk[a + r];
            }
        }
#pragma unroll
        for (int q = 0; q < kQ; ++q) {
            const int i = 4 * (q * NT + tid);
            f4a v = {0.0f, 0.0f, 0.0f, 0.0f};
            if (LOAD) {
                if (cnt == kOutTile) {
                    v = __builtin_nontemporal_load((const f4a*)(src + lo + i));
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        if (i + j < cnt) v[j] = src[lo + i + j];
                }
            }
            ini[q] = v;
        }
    };

    // prologue: entry ranges of tiles 0 and 1 of the sequence, the entries of
    // tile 0 in flight.  A tile's range is [ts(t), ts(t + 1)).
    const int32_t a0 = ts(tile(0)), e0 = ts(tile(0) + 1);
    int32_t a_nxt = ts(tile(1)), e_nxt = ts(tile(1) + 1);  // tile 1 (past the end: empty)
    if (ml == 0 && mk < kMerge) {
        S.a[0][mk] = a0;
        S.cnt[0][mk] = span(a0, e0);
    }
    clear_mask<NT>(S.mask);
    load_tile(tile(0), a0, span(a0, e0));
    __syncthreads();
    if (tid < 64) tile_meta<NT>(S, 0, 0, M.n, kPre * tpm);

    for (int64_t j = 0; j < J; ++j) {
        const int64_t u = tile(j);
        const int b = (int)(j & 1), z = (int)(j % 3);
        const int64_t lo = u * kOutTile;
        const int32_t cnt = (int32_t)min((int64_t)kOutTile, n - lo);
        // the previous tile (always whole) leaves LDS for memory; tile u's initial contents enter
#pragma unroll
        for (int q = 0; q < kQ; ++q) {
            const int i = 4 * (q * NT + tid);
            const f4a pt = *(const f4a*)(S.tile + i);
            *(f4a*)(S.tile + i) = ini[q];
            if (j > 0) __builtin_nontemporal_store(pt, (f4a*)(out + tile(j - 1) * kOutTile + i));
        }
        // this tile's entries, out of the pipeline registers, mark their messages
        int32_t ck[kPre], cp[kPre];
        float cv[kPre];
#pragma unroll
        for (int i = 0; i < kPre; ++i) {
            ck[i] = mk;
            cp[i] = (uint32_t)n_pos[i] < (uint32_t)cnt ? n_pos[i] : -1;  // always inside, for a clean message
            cv[i] = n_val[i];
        }
        mark_entries(S.mask, ck, cp);
        // the next tile in flight (its entries and initial contents), and the
        // range bounds of the one after it (clamped at the end of the iteration)
        const int64_t t2 = tile(j + 2);
        const int32_t r2a = ts_load(t2), r2e = ts_load(t2 + 1);
        if (j + 1 < J) {
            if (ml == 0 && mk < kMerge) {
                S.a[b ^ 1][mk] = a_nxt;
                S.cnt[b ^ 1][mk] = span(a_nxt, e_nxt);
            }
            load_tile(tile(j + 1), a_nxt, span(a_nxt, e_nxt));
        }
        __syncthreads();
        const int32_t total = S.total[z], fits = S.fits[z];  // uniform
        if (tid < 64 && j + 1 < J) tile_meta<NT>(S, b ^ 1, (int)((j + 1) % 3), M.n, kPre * tpm);
        if (total == 0) {
            // nothing to add (and nothing was marked)
        } else if (fits) {
            add_entries<NT>(S, S.mask, z, ck, cp, cv);
        } else {
            // from memory, kRound entries at a time in message order
            clear_mask<NT>(S.mask);  // drop the marks of the prefetched share
            __syncthreads();
            for (int32_t R0 = 0; R0 < total; R0 += kRound) {
#pragma unroll
                for (int i = 0; i < kPre; ++i) {
                    const int32_t e = R0 + tid + i * NT;
                    cp[i] = -1;
                    ck[i] = 0;
                    cv[i] = 0.0f;
                    if (e >= total) continue;
                    int32_t k = 0, off = 0;
                    while (e >= off + S.cnt[b][k]) off += S.cnt[b][k++];
                    const int32_t j = S.a[b][k] + (e - off);
                    const int32_t q = M.pos[k][j];
                    ck[i] = k;
                    cp[i] = (uint32_t)q < (uint32_t)cnt ? q : -1;
                    cv[i] = M.val[k][j];
                }
                mark_entries(S.mask, ck, cp);
                __syncthreads();
                add_entries<NT>(S, S.mask, z, ck, cp, cv);
                __syncthreads();  // mask cleared, depth read: the next round may start
                if (tid == 0) S.maxc[z] = 1;
            }
        }
        a_nxt = ts_fix(t2, r2a);
        e_nxt = ts_fix(t2 + 1, r2e);
    }
    __syncthreads();
    // the last tile
    const int64_t lo = tile(J - 1) * kOutTile;
    const int32_t cnt = (int32_t)min((int64_t)kOutTile, n - lo);
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
        const int i = 4 * (q * NT + tid);
        const f4a r = *(const f4a*)(S.tile + i);
        if (cnt == kOutTile) {
            __builtin_nontemporal_store(r, (f4a*)(out + lo + i));
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (i + j < cnt) out[lo + i + j] = r[j];
        }
    }
}

}  // namespace sgc

using namespace sgc;

// Persistent merge workgroups: as many as are resident at once on the device.
template <bool LOAD, int NT>
static int64_t merge_blocks()
{
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_merge<LOAD, NT>, NT, 0) != hipSuccess || cus <= 0 || per_cu <= 0)
        return 1024;
    return (int64_t)cus * per_cu;
}

static bool msg_ok(const sgc_layout* L, const sgc_message& m)
{
    if (m.format < SGC_MSG_RAW_F32 || m.format > SGC_MSG_GOLOMB_2BIT) return false;
    if (m.cap < 0 || m.cap >= ((int64_t)1 << 31) || !m.counts) return false;
    const bool nonempty = m.cap > 0;
    if (!is_golomb(m.format) && nonempty && !m.idx) return false;
    if ((m.format == SGC_MSG_RAW_F32 || m.format == SGC_MSG_GOLOMB_F32) && nonempty && !m.val) return false;
    if (is_2bit(m.format) && nonempty && (!m.codes || !m.means)) return false;
    if (m.format == SGC_MSG_GOLOMB_SBC && !m.means) return false;
    if (is_golomb(m.format)) {
        if (m.scope != SGC_GLOBAL && m.scope != SGC_PER_SEGMENT) return false;
        if (m.rice_b < 0 || m.rice_b > 30) return false;
        if (!m.word_off || !m.nbits || (nonempty && (!m.words || !m.chunk_off))) return false;
    }
    (void)L;
    return true;
}

extern "C" size_t sgc_decode_accumulate_workspace(const sgc_layout* L, const sgc_message* msgs, int32_t W)
{
    if (!L || W < 0 || (W > 0 && !msgs)) return 0;
    Carver c(nullptr);
    for (int32_t i = 0; i < W; ++i) {
        if (!msg_ok(L, msgs[i])) return 0;
        MsgWs w;
        carve_msg(c, L, msgs[i], &w);
    }
    return c.off;
}

extern "C" int sgc_decode_accumulate(const sgc_layout* Lc, const sgc_message* msgs, int32_t W, int32_t init,
                                     const float* base, float* out, uint32_t* dstatus, void* ws, size_t ws_bytes,
                                     sgc_stream_t stream)
{
    sgc_layout* L = const_cast<sgc_layout*>(Lc);
    if (!L || W < 0 || (W > 0 && !msgs)) return SGC_EINVAL;
    if (init != SGC_INIT_ZERO && init != SGC_INIT_BASE && init != SGC_INIT_INPLACE) return SGC_EINVAL;
    if (L->n > 0 && (!out || !aligned16(out))) return SGC_EINVAL;
    if (init == SGC_INIT_BASE && L->n > 0 && (!base || !aligned16(base))) return SGC_EINVAL;
    for (int32_t i = 0; i < W; ++i)
        if (!msg_ok(L, msgs[i])) return SGC_EINVAL;
    {
        Carver c0(nullptr);
        for (int32_t i = 0; i < W; ++i) {
            MsgWs w;
            carve_msg(c0, L, msgs[i], &w);
        }
        if (W > 0 && (!ws || ws_bytes < c0.off)) return SGC_ENOSPC;
    }
    if (L->n == 0) return SGC_OK;
    DevTables* dt = nullptr;
    int rc = device_tables(L, &dt);
    if (rc) return rc;
    hipStream_t s = (hipStream_t)stream;
    const int64_t ntiles = out_tiles(L);
    Carver c(ws);
    std::vector<MsgWs> mws((size_t)W);
    for (int32_t i = 0; i < W; ++i) carve_msg(c, L, msgs[i], &mws[(size_t)i]);

    for (int32_t b0 = 0; b0 < W; b0 += kBatch) {
        Batch B;
        B.n = std::min<int32_t>(kBatch, W - b0);
        int64_t maxcap = 0, maxch = 0;
        bool any_raw = false, any_2bit = false;
        int colw = 0;
        for (int32_t k = 0; k < B.n; ++k) {
            const sgc_message& m = msgs[b0 + k];
            MsgIn& in = B.in[k];
            in.format = m.format;
            in.scope = m.scope;
            in.b = m.rice_b;
            in.S = msg_streams(L, m);
            in.cap = m.cap;
            in.wbound = is_golomb(m.format) ? sgc_encode_word_bound(L, m.scope, m.rice_b, m.cap) : 0;
            in.counts = m.counts;
            in.idx = m.idx;
            in.val = m.val;
            in.codes = m.codes;
            in.means = m.means;
            in.words = m.words;
            in.word_off = m.word_off;
            in.nbits = m.nbits;
            in.chunk_off = m.chunk_off;
            B.ws[k] = mws[(size_t)(b0 + k)];
            maxcap = std::max(maxcap, m.cap);
            any_raw |= !is_golomb(m.format);
            any_2bit |= m.format == SGC_MSG_GOLOMB_2BIT;
            if (is_golomb(m.format)) colw = std::max(colw, col_words_for(m.rice_b));
            maxch = std::max(maxch, msg_nch(L, m));
        }
        const dim3 gtile((unsigned)std::max<int64_t>(1, std::min<int64_t>(cdiv(ntiles, kBlock), 2048)), (unsigned)B.n);
        k_msg_setup<<<gtile, kBlock, 0, s>>>(B, dt->seg_off, L->nseg, ntiles);
        SGC_LAUNCH_CHECK();
        const dim3 gch((unsigned)std::max<int64_t>(1, std::min<int64_t>(cdiv(maxch, kDecLanes), 16384)), (unsigned)B.n);
        if (any_2bit) launch_decode<true>(colw, gch, B, L->nseg, ntiles, s);
        else launch_decode<false>(colw, gch, B, L->nseg, ntiles, s);
        SGC_LAUNCH_CHECK();
        if (any_raw) {
            const dim3 gent((unsigned)std::max<int64_t>(1, std::min<int64_t>(cdiv(maxcap, kBlock * kEntPer), 4096)),
                            (unsigned)B.n);
            k_msg_entries<<<gent, kBlock, 0, s>>>(B, L->nseg, L->n, ntiles);
            SGC_LAUNCH_CHECK();
        }
        const dim3 gfill((unsigned)cdiv(ntiles, kFillTiles), (unsigned)B.n);
        k_fill_max<<<gfill, kBlock, 0, s>>>(B, ntiles);
        SGC_LAUNCH_CHECK();
        k_fill<<<gfill, kBlock, 0, s>>>(B, ntiles);
        SGC_LAUNCH_CHECK();
    }
    // merge in fixed message order; later batches continue in place
    const int64_t nmb = std::max<int64_t>(1, cdiv(W, kMerge));
    for (int64_t mb = 0; mb < nmb; ++mb) {
        MergeBatch M;
        const int32_t b0 = (int32_t)(mb * kMerge);
        M.n = std::min<int32_t>(kMerge, W - b0);
        for (int32_t k = 0; k < M.n; ++k) {
            const MsgWs& w = mws[(size_t)(b0 + k)];
            const sgc_message& mg = msgs[b0 + k];
            M.pos[k] = w.pos;
            M.val[k] = (mg.format == SGC_MSG_RAW_F32 || mg.format == SGC_MSG_GOLOMB_F32) ? mg.val : w.val;
            M.tstart[k] = w.tstart;
            M.bad[k] = w.bad;
        }
        // sparse batch (by the messages' capacities): 512 threads per workgroup
        int64_t capsum = 0;
        for (int32_t k = 0; k < M.n; ++k) capsum += msgs[b0 + k].cap;
        const bool sparse = capsum <= kMergeSparseEntries * ntiles;
        const int32_t nt = sparse ? 512 : 256;
        // threads per message slot: the workgroup / (message count rounded up to a power of two)
        int32_t lg_tpm = 0;
        while ((1 << (lg_tpm + 1)) <= nt) ++lg_tpm;
        while (lg_tpm > 0 && (nt >> lg_tpm) < M.n) --lg_tpm;
        const int32_t im = mb == 0 ? init : SGC_INIT_INPLACE;
        const bool load = im != SGC_INIT_ZERO;
        const int64_t resident = load ? (sparse ? merge_blocks<true, 512>() : merge_blocks<true, 256>())
                                      : (sparse ? merge_blocks<false, 512>() : merge_blocks<false, 256>());
        const int64_t grid = std::max<int64_t>(1, std::min<int64_t>(cdiv(ntiles, kTileRun), resident));
        uint32_t* st = M.n > 0 ? dstatus : nullptr;
        if (load && sparse)
            k_merge<true, 512><<<(unsigned)grid, 512, 0, s>>>(M, lg_tpm, im, base, out, L->n, ntiles, st);
        else if (load)
            k_merge<true, 256><<<(unsigned)grid, 256, 0, s>>>(M, lg_tpm, im, base, out, L->n, ntiles, st);
        else if (sparse)
            k_merge<false, 512><<<(unsigned)grid, 512, 0, s>>>(M, lg_tpm, im, base, out, L->n, ntiles, st);
        else
            k_merge<false, 256><<<(unsigned)grid, 256, 0, s>>>(M, lg_tpm, im, base, out, L->n, ntiles, st);
        SGC_LAUNCH_CHECK();
    }
    return SGC_OK;
}
