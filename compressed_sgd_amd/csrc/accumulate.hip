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
//  gaps    output-tile table entries for stretches no entry reaches;
//  raw     check that raw positions ascend; resolve 2-bit values;
//  decode  Rice streams: one thread per 256-code chunk starts from its
//          chunk-table entry (bit offset, position reached), decodes from
//          a copy of its words in LDS, writes global positions (and
//          resolved SBC / 2-bit values), and checks that it ends exactly
//          where the next chunk's entry says (or at the stream's bit count).
// Every message then has a sorted position list (its own idx if raw), a
// value list (its own val if fp32) and, per output tile, the index of its
// first entry at or beyond the tile.  The merge then gives
// each output tile to one workgroup: the initial tile and every message's
// entries for it are loaded in parallel, each thread applies the messages
// in order to the elements it owns (no atomics), and the tile is stored
// once: the dense output is written exactly once, in a fixed order.
#include "sgc_common.h"

namespace sgc {

typedef float f4a __attribute__((ext_vector_type(4)));

constexpr int kBatch = 8;     // messages per decode launch
constexpr int kMerge = 32;    // messages per merge launch

struct MsgWs {
    int64_t* estart;  // [nseg+1] entry prefix per segment
    int64_t* scnt;    // [S] codes per stream
    int64_t* sent;    // [S+1] first entry per stream
    int64_t* sbase;   // [S] first element of each stream
    int64_t* ssize;   // [S]
    int64_t* chpre;   // [S+1] chunk prefix
    int32_t* pos;     // [cap] decoded global positions
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
    const int32_t* pos[kMerge];
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
    w->pos = c.take<int32_t>(m.cap);
    w->val = c.take<float>(m.cap);
    w->tstart = c.take<int32_t>(out_tiles(L) + 1);
    w->bad = c.take<uint32_t>(1);
    w->total = c.take<int64_t>(1);
}

// ------------------------------------------------------------------ setup
__global__ void k_msg_setup(Batch B, const int64_t* __restrict__ seg_off, int32_t nseg, int64_t ntiles)
{
    if (threadIdx.x) return;
    const int m = blockIdx.y;
    const MsgIn& in = B.in[m];
    const MsgWs& w = B.ws[m];
    const int64_t n = seg_off[nseg];
    uint32_t bad = 0;
    int64_t e = 0;
    for (int32_t t = 0; t < nseg; ++t) {
        w.estart[t] = e;
        int64_t c = in.counts[t];
        if (c < 0 || c > in.cap - e) bad = 1;
        else e += c;
    }
    w.estart[nseg] = e;
    if (bad || in.counts[nseg] != e) bad = 1;
    const bool golomb = in.format >= SGC_MSG_GOLOMB_F32;
    int64_t ch = 0, se = 0;
    uint64_t wprev = 0;
    for (int32_t s = 0; s < in.S && !bad; ++s) {
        const bool glob = !golomb || in.scope == SGC_GLOBAL;
        const int64_t cnt = glob ? e : w.estart[s + 1] - w.estart[s];
        w.scnt[s] = cnt;
        w.sent[s] = se;
        w.sbase[s] = glob ? 0 : seg_off[s];
        w.ssize[s] = glob ? n : seg_off[s + 1] - seg_off[s];
        w.chpre[s] = ch;
        if (cnt > w.ssize[s]) bad = 1;
        if (golomb) {
            const uint64_t w0 = in.word_off[s], w1 = in.word_off[s + 1];
            if (w0 != wprev || w1 < w0 || (w1 - w0) != (in.nbits[s] + 31) / 32 || w1 > (uint64_t)in.wbound) bad = 1;
            if ((cnt > 0) != (in.nbits[s] > 0)) bad = 1;  // codes take at least one bit each; no codes, no bits
            wprev = w1;
        }
        se += cnt;
        ch += golomb ? cdiv(cnt, (int64_t)SGC_CHUNK_CODES) : 0;
    }
    if (bad) {
        for (int32_t s = 0; s < in.S; ++s) {
            w.scnt[s] = 0;
            w.sent[s] = 0;
            w.chpre[s] = 0;
        }
        ch = 0;
        se = 0;
    }
    w.sent[in.S] = se;
    w.chpre[in.S] = ch;
    w.bad[0] = bad;
    w.total[0] = bad ? 0 : e;
    w.tstart[ntiles] = (int32_t)(bad ? 0 : e);
}

// Output-tile table: entry j owns tiles (tile(prev), tile(pos)] -- the tiles
// whose first element lies after the previous entry and at or before it.
__device__ inline void fill_tiles(int32_t* tstart, int64_t from_pos_excl, int64_t to_pos_incl, int64_t j)
{
    const int64_t t0 = from_pos_excl < 0 ? 0 : from_pos_excl / kOutTile + 1;
    const int64_t t1 = to_pos_incl / kOutTile;
    for (int64_t t = t0; t <= t1; ++t) tstart[t] = (int32_t)j;
}

// ----------------------------------------------------------- raw messages
__global__ __launch_bounds__(kBlock) void k_msg_raw(Batch B, int32_t nseg, int64_t n, int64_t ntiles)
{
    const int m = blockIdx.y;
    const MsgIn& in = B.in[m];
    const MsgWs& w = B.ws[m];
    if (in.format >= SGC_MSG_GOLOMB_F32) return;
    const int64_t total = w.total[0];
    bool bad = false;
    for (int64_t j = (int64_t)blockIdx.x * kBlock + threadIdx.x; j < total; j += (int64_t)gridDim.x * kBlock) {
        const int64_t p = in.idx[j];
        const int64_t prev = j == 0 ? -1 : (int64_t)in.idx[j - 1];
        if (p < 0 || p >= n || p <= prev) { bad = true; continue; }
        if (in.format == SGC_MSG_RAW_2BIT) {  // RAW_F32: the merge reads idx/val directly
            const uint32_t code = (in.codes[j >> 4] >> (2 * (j & 15))) & 3u;
            const int64_t t = find_bucket(w.estart, (int64_t)nseg + 1, j);
            if (code == 3u) bad = true;
            w.val[j] = code == 0u ? 0.0f : code == 1u ? in.means[2 * t] : in.means[2 * t + 1];
        }
        fill_tiles(w.tstart, prev, p, j);
        if (j == total - 1) fill_tiles(w.tstart, p, n - 1, total);
    }
    if (bad) atomicOr(w.bad, 1u);
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
// whose words do not fit the column (very long gaps) decodes from global
// memory instead.  Positions (and, for SBC / 2-bit, resolved values) are
// buffered kDB at a time and stored together; the output-tile table is
// filled on the way, and the chunk is checked against its neighbours in
// the chunk table.
constexpr int kDB = 16;
constexpr int kDecLanes = 64;
constexpr int kColWords = 120;  // LDS words per lane (the chunk's words plus slack)
constexpr int kColCodes = 17;   // 2-bit code words per lane (256 entries span at most 17)

struct LdsWords {
    const uint32_t* col;  // this lane's column: col[i * kDecLanes]
    uint64_t w0, nw;      // first stream word held, words held
    __device__ uint32_t operator()(uint64_t i) const
    {
        const uint64_t r = i - w0;
        return r < nw ? col[r * kDecLanes] : 0u;
    }
};

struct GlobalWords {
    const uint32_t* w;
    uint64_t nw;
    __device__ uint32_t operator()(uint64_t i) const { return i < nw ? w[i] : 0u; }
};

// Sequential reader of one Rice stream over a word source; every read is
// checked against nbits.
template <typename Src>
struct WordReader {
    Src src;
    uint64_t nbits, pos, buf, wi;  // buf holds bits [pos, pos + avail); wi: next word to append
    uint32_t avail;
    __device__ void start(Src s, uint64_t nb, uint64_t bit)
    {
        src = s;
        nbits = nb;
        pos = bit;
        wi = (bit >> 5) + 1;
        const uint32_t sh = (uint32_t)(bit & 31);
        buf = (uint64_t)(src(bit >> 5) >> sh);
        avail = 32 - sh;
    }
    __device__ void refill()
    {
        while (avail <= 32) {
            buf |= (uint64_t)src(wi++) << avail;
            avail += 32;
        }
    }
    __device__ void consume(uint32_t k)
    {
        buf = k >= 64 ? 0ull : buf >> k;
        avail -= k;
        pos += k;
    }
    __device__ bool next(uint32_t b, uint64_t* z)
    {
        uint64_t q = 0;
        for (;;) {
            if (pos >= nbits) return false;
            refill();
            const uint64_t inv = ~buf;  // buf is 0 above avail, so the count stops at avail
            const uint32_t ones = inv ? (uint32_t)__builtin_ctzll(inv) : 64u;
            if (ones < avail) {
                if (pos + ones >= nbits) return false;
                q += ones;
                consume(ones + 1);
                break;
            }
            q += avail;
            consume(avail);
        }
        uint64_t rem = 0;
        if (b) {
            refill();
            if (pos + b > nbits) return false;
            rem = buf & ((1ull << b) - 1ull);
            consume(b);
        }
        if (q >> 33) return false;  // no stream is that long
        *z = (q << b) | rem;
        return true;
    }
};

// Decode one chunk with reader rd; returns false if the chunk is corrupt.
template <typename Rd>
__device__ inline bool decode_chunk(Rd& rd, const MsgIn& in, const MsgWs& w, const ChunkAt& a, int64_t c,
                                    int32_t nseg, uint64_t reached, const uint32_t* code_col)
{
    const int fmt = in.format;
    const int64_t size = w.ssize[a.s];
    const int64_t base = w.sbase[a.s];
    const int64_t j0 = w.sent[a.s] + a.q0;
    int64_t prev = (int64_t)reached - 1;
    // segment of the current entry (per-segment values), where its entries end, and its means
    int64_t t = in.scope == SGC_PER_SEGMENT ? a.s : find_bucket(w.estart, (int64_t)nseg + 1, j0);
    int64_t tend = in.scope == SGC_PER_SEGMENT ? INT64_MAX : w.estart[t + 1];
    float m0 = 0.0f, m1 = 0.0f;
    if (fmt == SGC_MSG_GOLOMB_SBC) m0 = in.means[t];
    if (fmt == SGC_MSG_GOLOMB_2BIT) {
        m0 = in.means[2 * t];
        m1 = in.means[2 * t + 1];
    }
    const bool values = fmt != SGC_MSG_GOLOMB_F32;  // F32 values are read by the merge directly
    int64_t gprev = base + prev;  // global position of the previous entry (tile table)
    for (int64_t i0 = 0; i0 < a.nc; i0 += kDB) {
        const int nb = (int)min((int64_t)kDB, a.nc - i0);
        int32_t pb[kDB];
        float vv[kDB];
#pragma unroll
        for (int q = 0; q < kDB; ++q) {
            pb[q] = 0;
            vv[q] = 0.0f;
            if (q >= nb) continue;
            uint64_t z;
            if (!rd.next((uint32_t)in.b, &z)) return false;
            const int64_t p = prev + 1 + (int64_t)z;
            if (p >= size) return false;
            prev = p;
            const int64_t j = j0 + i0 + q;
            while (j >= tend) {  // entered the next segment (global scope): rare
                ++t;
                tend = w.estart[t + 1];
                if (fmt == SGC_MSG_GOLOMB_SBC) m0 = in.means[t];
                if (fmt == SGC_MSG_GOLOMB_2BIT) {
                    m0 = in.means[2 * t];
                    m1 = in.means[2 * t + 1];
                }
            }
            if (fmt == SGC_MSG_GOLOMB_SBC) {
                vv[q] = m0;
            } else if (fmt == SGC_MSG_GOLOMB_2BIT) {
                const int64_t cw = (j >> 4) - (j0 >> 4);
                const uint32_t word = code_col ? code_col[cw * kDecLanes] : in.codes[j >> 4];
                const uint32_t code = (word >> (2 * (j & 15))) & 3u;
                if (code == 3u) return false;
                vv[q] = code == 0u ? 0.0f : code == 1u ? m0 : m1;
            }
            pb[q] = (int32_t)(base + p);
        }
        const int64_t jb = j0 + i0;
        if (nb == kDB && (jb & 3) == 0) {  // whole 64-byte sectors: four 16-byte stores per array
            typedef int32_t i4v __attribute__((ext_vector_type(4)));
#pragma unroll
            for (int q = 0; q < kDB / 4; ++q) {
                *(i4v*)(w.pos + jb + 4 * q) = i4v{pb[4 * q], pb[4 * q + 1], pb[4 * q + 2], pb[4 * q + 3]};
                if (values) *(f4a*)(w.val + jb + 4 * q) = f4a{vv[4 * q], vv[4 * q + 1], vv[4 * q + 2], vv[4 * q + 3]};
            }
        } else {
#pragma unroll
            for (int q = 0; q < kDB; ++q) {
                if (q >= nb) continue;
                w.pos[jb + q] = pb[q];
                if (values) w.val[jb + q] = vv[q];
            }
        }
#pragma unroll
        for (int q = 0; q < kDB; ++q) {
            if (q >= nb) continue;
            fill_tiles(w.tstart, gprev, pb[q], jb + q);
            gprev = pb[q];
        }
    }
    if (c + 1 < w.chpre[a.s + 1]) {
        // the next chunk must start exactly where this one ended
        if (in.chunk_off[2 * (c + 1)] != rd.pos || in.chunk_off[2 * (c + 1) + 1] != (uint64_t)(prev + 1)) return false;
    } else {
        if (rd.pos != rd.nbits) return false;  // no bits left over
        // the stream's last entry covers the tiles up to the end of its range
        fill_tiles(w.tstart, gprev, base + size - 1, w.sent[a.s + 1]);
    }
    return true;
}

__global__ __launch_bounds__(kDecLanes) void k_msg_decode(Batch B, int32_t nseg, int64_t n)
{
    __shared__ uint32_t col[kColWords * kDecLanes];
    __shared__ uint32_t ccol[kColCodes * kDecLanes];
    const int m = blockIdx.y;
    const MsgIn& in = B.in[m];
    const MsgWs& w = B.ws[m];
    if (in.format < SGC_MSG_GOLOMB_F32) return;
    if (w.bad[0]) return;
    const int lane = threadIdx.x;
    const int64_t nch = w.chpre[in.S];
    bool bad = false;
    for (int64_t c = (int64_t)blockIdx.x * kDecLanes + lane; c < nch; c += (int64_t)gridDim.x * kDecLanes) {
        const ChunkAt a = chunk_at(w, in.S, c);
        const uint64_t bit0 = in.chunk_off[2 * c], reached = in.chunk_off[2 * c + 1];
        if ((a.q0 == 0 && (bit0 != 0 || reached != 0)) || reached > (uint64_t)w.ssize[a.s]) { bad = true; continue; }
        const uint32_t* words = in.words + in.word_off[a.s];
        const uint64_t nw = in.word_off[a.s + 1] - in.word_off[a.s];
        const uint64_t nbits = in.nbits[a.s];
        const uint64_t bit1 = (c + 1 < w.chpre[a.s + 1]) ? in.chunk_off[2 * (c + 1)] : nbits;
        if (bit1 < bit0 || bit1 > nbits) { bad = true; continue; }
        // 2-bit code words of the chunk's entries
        const uint32_t* code_col = nullptr;
        if (in.format == SGC_MSG_GOLOMB_2BIT) {
            const int64_t j0 = w.sent[a.s] + a.q0;
            const int64_t cw0 = j0 >> 4, cw1 = (j0 + a.nc - 1) >> 4;
#pragma unroll 4
            for (int64_t i = 0; i <= cw1 - cw0; ++i) ccol[i * kDecLanes + lane] = in.codes[cw0 + i];
            code_col = ccol + lane;
        }
        // words [bit0/32, bit1/32 + 2): the chunk's bits plus a two-word window slack
        const uint64_t wlo = bit0 >> 5;
        const uint64_t whi = min((bit1 >> 5) + 2, nw);
        const uint64_t nwc = whi > wlo ? whi - wlo : 0;
        bool ok;
        if (nwc <= (uint64_t)kColWords) {
#pragma unroll 8
            for (uint64_t i = 0; i < nwc; ++i) col[i * kDecLanes + lane] = words[wlo + i];
            WordReader<LdsWords> rd;
            rd.start(LdsWords{col + lane, wlo, nwc}, nbits, bit0);
            ok = decode_chunk(rd, in, w, a, c, nseg, reached, code_col);
        } else {
            WordReader<GlobalWords> rd;
            rd.start(GlobalWords{words, nw}, nbits, bit0);
            ok = decode_chunk(rd, in, w, a, c, nseg, reached, code_col);
        }
        if (!ok) bad = true;
    }
    if (bad) atomicOr(w.bad, 1u);
}

// Tiles that start inside a stream without entries: the first entry at or
// beyond them is the next stream's first entry.
__global__ __launch_bounds__(kBlock) void k_msg_gaps(Batch B, int64_t n, int64_t ntiles)
{
    const int m = blockIdx.y;
    const MsgIn& in = B.in[m];
    const MsgWs& w = B.ws[m];
    for (int64_t t = (int64_t)blockIdx.x * kBlock + threadIdx.x; t < ntiles; t += (int64_t)gridDim.x * kBlock) {
        const int64_t p = t * kOutTile;
        int64_t s = 0;
        if (in.S > 1) {
            // stream containing element p (streams are the segments, in order)
            int64_t lo = 0, hi = in.S - 1;
            while (lo < hi) {
                const int64_t mid = (lo + hi + 1) >> 1;
                if (w.sbase[mid] <= p) lo = mid; else hi = mid - 1;
            }
            s = lo;
            while (s + 1 < in.S && w.ssize[s] == 0 && w.sbase[s + 1] <= p) ++s;
        }
        if (w.scnt[s] == 0) w.tstart[t] = (int32_t)w.sent[s];
    }
}

// ------------------------------------------------------------------ merge
// One workgroup per output tile of kOutTile elements.  Round 1 (parallel):
// the tile's initial contents (coalesced, into LDS) and every message's
// entry range [tstart[t], tstart[t+1]).  Then the entries of all messages
// are staged in LDS (kStage at a time, in message order) and thread t
// applies, for each message in order, the entries that fall on the 16
// contiguous tile elements it owns (binary search in the staged, ascending
// positions).  No element is touched by two threads, so there are no
// atomics and no per-message barriers; the tile is stored once, coalesced.
constexpr int kStage = 1024;
constexpr int kOwn = (int)(kOutTile / kBlock);  // 16 elements per thread

__global__ __launch_bounds__(kBlock) void k_merge(MergeBatch M, int32_t init, const float* __restrict__ base,
                                                 float* __restrict__ out, int64_t n)
{
    __shared__ float tile[kOutTile];
    __shared__ int32_t s_a[kMerge], s_off[kMerge + 1];
    __shared__ uint16_t st_pos[kStage];
    __shared__ float st_val[kStage];
    const int64_t t = blockIdx.x;
    const int64_t lo = t * kOutTile;
    const int64_t cnt = min((int64_t)kOutTile, n - lo);
    const bool full = cnt == kOutTile;
    constexpr int kQ = (int)(kOutTile / (4 * kBlock));
    if (threadIdx.x < 64) {  // wave 0: message ranges and their prefix
        const int k = threadIdx.x;
        int32_t a = 0, c = 0;
        if (k < M.n && !*M.bad[k]) {
            a = M.tstart[k][t];
            c = M.tstart[k][t + 1] - a;
        }
        int32_t x = c;
        for (int d = 1; d < 64; d <<= 1) {
            const int32_t y = __shfl_up(x, d, 64);
            if (k >= d) x += y;
        }
        if (k < kMerge) {
            s_a[k] = a;
            s_off[k] = x - c;
        }
        if (k == kMerge - 1) s_off[kMerge] = x;
    }
    {
        const float* src = init == SGC_INIT_BASE ? base : out;
#pragma unroll
        for (int q = 0; q < kQ; ++q) {
            const int i = 4 * (q * kBlock + threadIdx.x);
            f4a v = {0.0f, 0.0f, 0.0f, 0.0f};
            if (init != SGC_INIT_ZERO) {
                if (full) {
                    v = *(const f4a*)(src + lo + i);
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        if (i + j < cnt) v[j] = src[lo + i + j];
                }
            }
            *(f4a*)(tile + i) = v;
        }
    }
    __syncthreads();
    const int own0 = threadIdx.x * kOwn;
    const int32_t total = s_off[kMerge];
    for (int32_t R0 = 0; R0 < total; R0 += kStage) {  // uniform; one round in the common case
        const int32_t R1 = min(R0 + kStage, total);
        for (int32_t e = R0 + threadIdx.x; e < R1; e += kBlock) {
            int k = 0;
            while (e >= s_off[k + 1]) ++k;
            const int32_t j = s_a[k] + (e - s_off[k]);
            const int64_t p = (int64_t)M.pos[k][j] - lo;
            st_pos[e - R0] = (uint16_t)((uint64_t)p < (uint64_t)cnt ? p : 0xffff);
            st_val[e - R0] = M.val[k][j];
        }
        __syncthreads();
        for (int k = 0; k < M.n; ++k) {
            const int32_t e0 = max(s_off[k], R0) - R0, e1 = min(s_off[k + 1], R1) - R0;
            if (e0 >= e1) continue;
            // first staged entry of message k at or after own0 (positions ascend)
            int32_t l = e0, h = e1;
            while (l < h) {
                const int32_t m = (l + h) >> 1;
                if ((int32_t)st_pos[m] < own0) l = m + 1; else h = m;
            }
            for (int32_t e = l; e < e1; ++e) {
                const int32_t p = st_pos[e];
                if (p >= own0 + kOwn) break;  // also stops at the 0xffff sentinel
                tile[p] = tile[p] + st_val[e];
            }
        }
        __syncthreads();  // staging is refilled by the next round; the tile is read below
    }
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
        const int i = 4 * (q * kBlock + threadIdx.x);
        const f4a r = *(const f4a*)(tile + i);
        if (full) {
            __builtin_nontemporal_store(r, (f4a*)(out + lo + i));
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (i + j < cnt) out[lo + i + j] = r[j];
        }
    }
}

__global__ void k_fold_status(MergeBatch M, uint32_t* status)
{
    if (threadIdx.x) return;
    uint32_t st = 0;
    for (int k = 0; k < M.n; ++k)
        if (*M.bad[k]) st |= SGC_STATUS_CORRUPT;
    if (st) *status |= st;
}

}  // namespace sgc

using namespace sgc;

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
            maxch = std::max(maxch, msg_nch(L, m));
        }
        const dim3 one(1, (unsigned)B.n);
        k_msg_setup<<<one, 64, 0, s>>>(B, dt->seg_off, L->nseg, ntiles);
        SGC_LAUNCH_CHECK();
        const dim3 gtile((unsigned)std::max<int64_t>(1, std::min<int64_t>(cdiv(ntiles, kBlock), 2048)), (unsigned)B.n);
        k_msg_gaps<<<gtile, kBlock, 0, s>>>(B, L->n, ntiles);
        SGC_LAUNCH_CHECK();
        const dim3 graw((unsigned)std::max<int64_t>(1, std::min<int64_t>(cdiv(maxcap, kBlock), 4096)), (unsigned)B.n);
        k_msg_raw<<<graw, kBlock, 0, s>>>(B, L->nseg, L->n, ntiles);
        SGC_LAUNCH_CHECK();
        const dim3 gch((unsigned)std::max<int64_t>(1, std::min<int64_t>(cdiv(maxch, kDecLanes), 16384)), (unsigned)B.n);
        k_msg_decode<<<gch, kDecLanes, 0, s>>>(B, L->nseg, L->n);
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
            M.pos[k] = is_golomb(mg.format) ? w.pos : mg.idx;
            M.val[k] = (mg.format == SGC_MSG_RAW_F32 || mg.format == SGC_MSG_GOLOMB_F32) ? mg.val : w.val;
            M.tstart[k] = w.tstart;
            M.bad[k] = w.bad;
        }
        k_merge<<<(unsigned)ntiles, kBlock, 0, s>>>(M, mb == 0 ? init : SGC_INIT_INPLACE, base, out, L->n);
        SGC_LAUNCH_CHECK();
        if (dstatus && M.n > 0) {
            k_fold_status<<<1, 64, 0, s>>>(M, dstatus);
            SGC_LAUNCH_CHECK();
        }
    }
    return SGC_OK;
}
