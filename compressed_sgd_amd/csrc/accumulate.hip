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
//  raw     copy positions and resolved values, check they ascend;
//  span    Rice streams: one thread per 256-code chunk decodes from the
//          chunk table and records the chunk's position span, checking
//          that it ends exactly where the next chunk starts;
//  scan    exclusive scan of spans -> position before every chunk;
//  decode  decode again, writing global positions and resolved values;
//  gaps    output-tile table entries for stretches no entry reaches.
// Every message leaves a sorted (pos, val) list and, per 4096-element
// output tile, the index of its first entry at or beyond the tile.  The
// merge then gives each output tile to one workgroup: the tile is loaded
// (or zeroed) into LDS, messages are applied in order (entries of one
// message have distinct positions, so no atomics), and the tile is stored
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
    uint64_t* span;   // [nch] position span of each chunk
    int64_t* cprev;   // [nch] stream-relative position before each chunk
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
    w->span = c.take<uint64_t>(nch);
    w->cprev = c.take<int64_t>(nch);
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
            if (cnt > 0 && in.nbits[s] == 0) bad = 1;
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
        float v;
        if (in.format == SGC_MSG_RAW_F32) {
            v = in.val[j];
        } else {
            const uint32_t code = (in.codes[j >> 4] >> (2 * (j & 15))) & 3u;
            const int64_t t = find_bucket(w.estart, (int64_t)nseg + 1, j);
            if (code == 3u) bad = true;
            v = code == 0u ? 0.0f : code == 1u ? in.means[2 * t] : in.means[2 * t + 1];
        }
        w.pos[j] = (int32_t)p;
        w.val[j] = v;
        fill_tiles(w.tstart, prev, p, j);
        if (j == total - 1) fill_tiles(w.tstart, p, n - 1, total);
    }
    if (bad) atomicOr(w.bad, 1u);
}

// --------------------------------------------------------- Rice decoding
struct Bits {
    const uint32_t* w;
    uint64_t nw, nbits;
    __device__ uint64_t window(uint64_t bit) const
    {
        const uint64_t i = bit >> 5;
        const uint32_t sh = (uint32_t)(bit & 31);
        const uint64_t a = i < nw ? w[i] : 0, b = i + 1 < nw ? w[i + 1] : 0, c = i + 2 < nw ? w[i + 2] : 0;
        const uint64_t lo = a | (b << 32);
        return sh ? (lo >> sh) | (c << (64 - sh)) : lo;
    }
    // Decode one code at *bit; returns false on a read past nbits.
    __device__ bool next(uint64_t* bit, uint32_t b, uint64_t* z) const
    {
        uint64_t q = 0, p = *bit;
        for (;;) {
            if (p >= nbits) return false;
            const uint64_t win = window(p);
            const uint64_t inv = ~win;
            if (inv) {
                const uint32_t ones = (uint32_t)__builtin_ctzll(inv);
                if (p + ones >= nbits) return false;
                q += ones;
                p += ones + 1;
                break;
            }
            q += 64;
            p += 64;
        }
        uint64_t rem = 0;
        if (b) {
            if (p + b > nbits) return false;
            rem = window(p) & ((1ull << b) - 1ull);
            p += b;
        }
        if (q >> 33) return false;  // no stream is that long
        *z = (q << b) | rem;
        *bit = p;
        return true;
    }
};

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

__device__ inline Bits stream_bits(const MsgIn& in, int64_t s)
{
    Bits r;
    r.w = in.words + in.word_off[s];
    r.nw = in.word_off[s + 1] - in.word_off[s];
    r.nbits = in.nbits[s];
    return r;
}

__global__ __launch_bounds__(kBlock) void k_msg_span(Batch B)
{
    const int m = blockIdx.y;
    const MsgIn& in = B.in[m];
    const MsgWs& w = B.ws[m];
    if (in.format < SGC_MSG_GOLOMB_F32) return;
    const int64_t nch = w.chpre[in.S];
    bool bad = false;
    for (int64_t c = (int64_t)blockIdx.x * kBlock + threadIdx.x; c < nch; c += (int64_t)gridDim.x * kBlock) {
        const ChunkAt a = chunk_at(w, in.S, c);
        const Bits bits = stream_bits(in, a.s);
        uint64_t bit = in.chunk_off[c];
        if (a.q0 == 0 && bit != 0) { bad = true; continue; }
        uint64_t span = 0, z;
        bool ok = true;
        for (int64_t i = 0; i < a.nc; ++i) {
            if (!bits.next(&bit, (uint32_t)in.b, &z)) { ok = false; break; }
            span += z + 1;
            if (span > (uint64_t)w.ssize[a.s]) { ok = false; break; }
        }
        const uint64_t want = (c + 1 < w.chpre[a.s + 1]) ? in.chunk_off[c + 1] : bits.nbits;
        if (!ok || bit != want) bad = true;
        w.span[c] = span;
    }
    if (bad) atomicOr(w.bad, 1u);
}

__global__ __launch_bounds__(1024) void k_msg_scan(Batch B)
{
    const int m = blockIdx.y;
    const MsgIn& in = B.in[m];
    const MsgWs& w = B.ws[m];
    if (in.format < SGC_MSG_GOLOMB_F32) return;
    __shared__ uint64_t tmp[1024 / 64 + 1];
    // flat exclusive scan of spans, then rebase per stream
    const int64_t nch = w.chpre[in.S];
    const int64_t per = cdiv(nch, (int64_t)blockDim.x);
    const int64_t b0 = threadIdx.x * per, e0 = min(b0 + per, nch);
    uint64_t local = 0;
    for (int64_t c = b0; c < e0; ++c) local += w.span[c];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint64_t x = local;
    for (int d = 1; d < 64; d <<= 1) {
        uint64_t y = __shfl_up(x, d, 64);
        if (lane >= d) x += y;
    }
    if (lane == 63) tmp[wave] = x;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint64_t run = 0;
        for (int i = 0; i < (int)(blockDim.x >> 6); ++i) { uint64_t q = tmp[i]; tmp[i] = run; run += q; }
    }
    __syncthreads();
    uint64_t run = tmp[wave] + x - local;
    for (int64_t c = b0; c < e0; ++c) {
        w.cprev[c] = (int64_t)run;  // flat prefix; chunk_prev() rebases it per stream
        run += w.span[c];
    }
}

// Position before chunk c, relative to its stream: -1 + (flat prefix of c) -
// (flat prefix of the stream's first chunk).
__device__ inline int64_t chunk_prev(const MsgWs& w, const ChunkAt& a, int64_t c)
{
    return -1 + w.cprev[c] - w.cprev[w.chpre[a.s]];
}

__global__ __launch_bounds__(kBlock) void k_msg_decode(Batch B, int32_t nseg, int64_t n)
{
    const int m = blockIdx.y;
    const MsgIn& in = B.in[m];
    const MsgWs& w = B.ws[m];
    if (in.format < SGC_MSG_GOLOMB_F32) return;
    if (w.bad[0]) return;
    const int64_t nch = w.chpre[in.S];
    bool bad = false;
    for (int64_t c = (int64_t)blockIdx.x * kBlock + threadIdx.x; c < nch; c += (int64_t)gridDim.x * kBlock) {
        const ChunkAt a = chunk_at(w, in.S, c);
        const Bits bits = stream_bits(in, a.s);
        uint64_t bit = in.chunk_off[c], z;
        int64_t prev = chunk_prev(w, a, c);
        const int64_t base = w.sbase[a.s];
        int64_t j = w.sent[a.s] + a.q0;
        // segment of entry j for per-segment values
        int64_t t = in.scope == SGC_PER_SEGMENT ? a.s : find_bucket(w.estart, (int64_t)nseg + 1, j);
        // the previous entry's global position (for the tile table)
        int64_t gprev = prev >= 0 ? base + prev : base - 1;
        for (int64_t i = 0; i < a.nc; ++i, ++j) {
            if (!bits.next(&bit, (uint32_t)in.b, &z)) { bad = true; break; }
            const int64_t p = prev + 1 + (int64_t)z;
            if (p >= w.ssize[a.s]) { bad = true; break; }
            prev = p;
            const int64_t gp = base + p;
            while (in.scope != SGC_PER_SEGMENT && j >= w.estart[t + 1]) ++t;
            float v;
            if (in.format == SGC_MSG_GOLOMB_F32) {
                v = in.val[j];
            } else if (in.format == SGC_MSG_GOLOMB_SBC) {
                v = in.means[t];
            } else {
                const uint32_t code = (in.codes[j >> 4] >> (2 * (j & 15))) & 3u;
                if (code == 3u) bad = true;
                v = code == 0u ? 0.0f : code == 1u ? in.means[2 * t] : in.means[2 * t + 1];
            }
            w.pos[j] = (int32_t)gp;
            w.val[j] = v;
            fill_tiles(w.tstart, gprev, gp, j);
            gprev = gp;
        }
        // the stream's last entry covers the tiles up to the end of its range
        if (!bad && a.q0 + a.nc == w.scnt[a.s])
            fill_tiles(w.tstart, gprev, base + w.ssize[a.s] - 1, w.sent[a.s + 1]);
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
__global__ __launch_bounds__(kBlock) void k_merge(MergeBatch M, int32_t init, const float* __restrict__ base,
                                                 float* __restrict__ out, int64_t n)
{
    __shared__ float tile[kOutTile];
    const int64_t t = blockIdx.x;
    const int64_t lo = t * kOutTile;
    const int64_t cnt = min((int64_t)kOutTile, n - lo);
    const bool full = cnt == kOutTile;
    // initial contents
    for (int q = 0; q < (int)(kOutTile / (4 * kBlock)); ++q) {
        const int i = 4 * (q * kBlock + threadIdx.x);
        f4a v = {0.0f, 0.0f, 0.0f, 0.0f};
        if (init != SGC_INIT_ZERO) {
            const float* src = init == SGC_INIT_BASE ? base : out;
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
    __syncthreads();
    for (int k = 0; k < M.n; ++k) {
        if (*M.bad[k]) continue;  // uniform per block
        const int32_t a = M.tstart[k][t], e = M.tstart[k][t + 1];
        for (int32_t j = a + threadIdx.x; j < e; j += kBlock) {
            const int64_t p = (int64_t)M.pos[k][j] - lo;
            if ((uint64_t)p < (uint64_t)cnt) tile[p] = tile[p] + M.val[k][j];
        }
        __syncthreads();
    }
    for (int q = 0; q < (int)(kOutTile / (4 * kBlock)); ++q) {
        const int i = 4 * (q * kBlock + threadIdx.x);
        const f4a v = *(const f4a*)(tile + i);
        if (full) {
            __builtin_nontemporal_store(v, (f4a*)(out + lo + i));
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (i + j < cnt) out[lo + i + j] = v[j];
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
        const dim3 gch((unsigned)std::max<int64_t>(1, std::min<int64_t>(cdiv(maxch, kBlock), 4096)), (unsigned)B.n);
        k_msg_span<<<gch, kBlock, 0, s>>>(B);
        SGC_LAUNCH_CHECK();
        k_msg_scan<<<one, 1024, 0, s>>>(B);
        SGC_LAUNCH_CHECK();
        k_msg_decode<<<gch, kBlock, 0, s>>>(B, L->nseg, L->n);
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
            M.pos[k] = w.pos;
            M.val[k] = w.val;
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
