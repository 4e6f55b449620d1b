// rice.hip -- Rice (power-of-two Golomb) coding of index gaps (sgc_encode).
//
// [SBC] §II Optimal Position Encoding: the distances between nonzero
// elements are Golomb coded instead of their positions.  [SBC] appendix A:
// both ends know the tensor shapes, so a stream carries no shape data.
//
// Code of a gap z (zeros skipped before the next entry) with parameter b:
// floor(z / 2^b) one-bits, a zero-bit, then the b low bits of z LSB-first.
// Stream bit i is bit (i mod 32) of the stream's word i / 32.
//
// GPU design: encode blocks of 2048 codes that never straddle a stream.
//  1. lengths: per block the sum of code lengths;
//  2. scan:    block bit offsets (flat scan), stream bit counts and word
//              offsets (streams start on word boundaries);
//  3. pack:    per block, code offsets by one block scan; every code ORs
//              its bits into an LDS copy of the output words whose first
//              bit lies in the block (plus up to 32 look-ahead codes of the
//              next block, which complete the last word), and the words are
//              stored once, coalesced: no global atomics, no pre-zeroing.
//              The chunk table (bit offset and position reached for every
//              256th code) is written on the way.
#include "sgc_common.h"

namespace sgc {

struct EncWs {
    int64_t* cnt;    // [S] codes per stream
    int64_t* ent;    // [S+1] first entry of each stream
    int64_t* base;   // [S] position of the stream's element 0
    int64_t* size;   // [S] elements covered by the stream
    int64_t* ebpre;  // [S+1] encode-block prefix
    int64_t* chpre;  // [S+1] chunk-table prefix
    uint64_t* ebits; // [neb] bits per encode block
    uint64_t* eboff; // [neb+1] flat exclusive prefix of ebits
    uint64_t* sbit0; // [S] flat bit offset of each stream's first block
    uint64_t* part;  // [neb_max / kScanPart + 1] bit totals per scan part (split scan only)
    uint32_t* bad;   // [1] malformed-input flags
    uint32_t* st;    // [1] status target when the caller passes none
};

// The block-offset scan runs in one workgroup up to kScanSplit encode
// blocks; beyond that (kept fractions of ~5% and up at 2^30 elements) one
// workgroup does too much shuffle work, and it is split over workgroups of
// kScanPart blocks each.
constexpr int64_t kScanPart = 4096;
constexpr int64_t kScanSplit = 16384;

static int32_t enc_streams(const sgc_layout* L, int32_t scope) { return scope == SGC_GLOBAL ? 1 : L->nseg; }
static int64_t enc_neb_max(const sgc_layout* L, int32_t scope, int64_t cap)
{
    return cdiv(cap, kEncCodes) + enc_streams(L, scope) + 1;
}

static void carve_enc(Carver& c, const sgc_layout* L, int32_t scope, int64_t cap, EncWs* w)
{
    const int64_t S = enc_streams(L, scope), neb = enc_neb_max(L, scope, cap);
    w->cnt = c.take<int64_t>(S);
    w->ent = c.take<int64_t>(S + 1);
    w->base = c.take<int64_t>(S);
    w->size = c.take<int64_t>(S);
    w->ebpre = c.take<int64_t>(S + 1);
    w->chpre = c.take<int64_t>(S + 1);
    w->ebits = c.take<uint64_t>(neb);
    w->eboff = c.take<uint64_t>(neb + 1);
    w->sbit0 = c.take<uint64_t>(S);
    w->part = c.take<uint64_t>(cdiv(neb, kScanPart) + 1);
    w->bad = c.take<uint32_t>(1);
    w->st = c.take<uint32_t>(1);
}

// Per-stream tables, one thread per stream in rounds (workgroup scans).
// Counts are clamped to the room left below cap (entry prefix = min(cap,
// prefix of the clamped counts)), so that malformed counts never move a
// read past cap entries; they are flagged.
__global__ __launch_bounds__(kBlock) void k_enc_setup(const int64_t* __restrict__ counts,
                                                     const int64_t* __restrict__ seg_off, int32_t nseg,
                                                     int32_t scope, int64_t cap, EncWs w)
{
    __shared__ int64_t tmp[kBlock / 64 + 1];
    const int32_t S = scope == SGC_GLOBAL ? 1 : nseg;
    int64_t P = 0, EB = 0, CH = 0;  // prefixes carried from round to round
    bool bad = false;
    for (int64_t s0 = 0; s0 < S; s0 += kBlock) {
        const int64_t s = s0 + threadIdx.x;
        const bool in = s < S;
        const int64_t raw = in ? (scope == SGC_GLOBAL ? counts[nseg] : counts[s]) : 0;
        const int64_t c = raw < 0 ? 0 : (raw > cap ? cap : raw);
        int64_t tp, teb, tch;
        const int64_t xp = P + block_scan_excl<kBlock, int64_t>(c, tmp, &tp);
        const int64_t e0 = xp < cap ? xp : cap, e1 = xp + c < cap ? xp + c : cap;
        const int64_t m = e1 - e0;
        bad |= in && (raw < 0 || raw > cap - e0);
        const int64_t xeb = EB + block_scan_excl<kBlock, int64_t>(cdiv(m, kEncCodes), tmp, &teb);
        const int64_t xch = CH + block_scan_excl<kBlock, int64_t>(cdiv(m, (int64_t)SGC_CHUNK_CODES), tmp, &tch);
        if (in) {
            w.cnt[s] = m;
            w.ent[s] = e0;
            w.base[s] = scope == SGC_GLOBAL ? 0 : seg_off[s];
            w.size[s] = scope == SGC_GLOBAL ? seg_off[nseg] : seg_off[s + 1] - seg_off[s];
            w.ebpre[s] = xeb;
            w.chpre[s] = xch;
        }
        P += tp;
        EB += teb;
        CH += tch;
    }
    bad = __syncthreads_or(bad);
    if (threadIdx.x == 0) {
        w.bad[0] = bad ? 1u : 0u;
        w.ent[S] = P < cap ? P : cap;
        w.ebpre[S] = EB;
        w.chpre[S] = CH;
    }
}

struct EncBlock {
    int64_t s, e0, e1, ahead;
};

__device__ inline EncBlock enc_block(const EncWs& w, int32_t S, int64_t b)
{
    EncBlock k;
    k.s = find_bucket(w.ebpre, (int64_t)S + 1, b);
    k.e0 = w.ent[k.s] + (b - w.ebpre[k.s]) * kEncCodes;
    k.e1 = min(k.e0 + kEncCodes, w.ent[k.s + 1]);
    k.ahead = min((int64_t)kEncAhead, w.ent[k.s + 1] - k.e1);
    return k;
}

// Gap before entry j of stream s, from its index and the index before it
// (loaded unconditionally from max(j-1, first entry); replaced here by the
// stream's origin for the first entry).  Flags malformed input (not strictly
// ascending, or outside the stream) and codes it as a zero gap.
struct EncStream {
    int64_t first, base, size;  // first entry, position of element 0, elements covered
};

__device__ inline EncStream enc_stream(const EncWs& w, int64_t s) { return {w.ent[s], w.base[s], w.size[s]}; }

__device__ inline uint32_t enc_gap(int32_t cur, int32_t before, const EncStream& st, int64_t j, bool* bad)
{
    const int64_t pos = (int64_t)cur - st.base;
    const int64_t prev = j == st.first ? -1 : (int64_t)before - st.base;
    const int64_t z = pos - prev - 1;
    if (z < 0 || pos >= st.size) {
        *bad = true;
        return 0;
    }
    return (uint32_t)z;
}

constexpr int kEncLenPer = (int)(kEncCodes / kBlock);  // codes per thread in the length pass
static_assert(kEncLenPer * kBlock == kEncCodes, "encode block = whole rounds of the workgroup");

__global__ __launch_bounds__(kBlock) void k_enc_len(const int32_t* __restrict__ idx, int32_t S, int32_t b, EncWs w)
{
    __shared__ uint64_t tmp[kBlock / 64 + 1];
    const int64_t neb = w.ebpre[S];
    for (int64_t blk = blockIdx.x; blk < neb; blk += gridDim.x) {
        const EncBlock k = enc_block(w, S, blk);
        const EncStream st = enc_stream(w, k.s);
        // clamped, unconditional loads: all in flight at once
        int32_t cur[kEncLenPer], bef[kEncLenPer];
#pragma unroll
        for (int q = 0; q < kEncLenPer; ++q) {
            const int64_t j = min(k.e0 + q * kBlock + threadIdx.x, k.e1 - 1);
            cur[q] = idx[j];
            bef[q] = idx[j > st.first ? j - 1 : j];
        }
        uint64_t bits = 0;
        bool bad = false;
#pragma unroll
        for (int q = 0; q < kEncLenPer; ++q) {
            const int64_t j = k.e0 + q * kBlock + threadIdx.x;
            if (j < k.e1) {
                const uint32_t z = enc_gap(cur[q], bef[q], st, j, &bad);
                bits += (uint64_t)(z >> b) + 1 + (uint64_t)b;
            }
        }
        if (bad) atomicOr(w.bad, 1u);
        uint64_t tot;
        block_exclusive_scan<uint64_t>(bits, tmp, &tot);
        if (threadIdx.x == 0) w.ebits[blk] = tot;
    }
}

constexpr int kEncScanU = 4;  // 64-entry steps per batch of loads in the block scan

// Exclusive prefix of the encode blocks' bit counts.  Each wave owns a
// contiguous range, a multiple of 64 entries long, and reads it 64
// consecutive entries per load (coalesced; a per-thread range would put
// every lane of a load on its own cache line); the range total first, then,
// after the wave offsets are known, a shuffle scan per step with a running
// carry.
// Split scan, part 1: the bit total of each part of kScanPart encode blocks
// (coalesced reads; parts past the end give 0).
__global__ __launch_bounds__(kBlock) void k_enc_scan_part(int32_t S, EncWs w)
{
    __shared__ uint64_t tmp[kBlock / 64 + 1];
    const int64_t neb = w.ebpre[S];
    const int64_t b0 = (int64_t)blockIdx.x * kScanPart, b1 = min(b0 + kScanPart, neb);
    uint64_t local = 0;
    for (int64_t i = b0 + threadIdx.x; i < b1; i += kBlock) local += w.ebits[i];
    uint64_t total;
    block_scan_excl<kBlock, uint64_t>(local, tmp, &total);
    if (threadIdx.x == 0) w.part[blockIdx.x] = total;
}

// Split scan, part 2: each workgroup adds up the parts before its own (a few
// dozen at most) and scans its part in rounds of kBlock, coalesced; the
// workgroup holding the last block writes the flat total.
__global__ __launch_bounds__(kBlock) void k_enc_scan_apply(int32_t S, EncWs w)
{
    __shared__ uint64_t tmp[kBlock / 64 + 1];
    const int64_t neb = w.ebpre[S];
    const int64_t b0 = (int64_t)blockIdx.x * kScanPart, b1 = min(b0 + kScanPart, neb);
    uint64_t before = 0;
    for (int64_t q = threadIdx.x; q < (int64_t)blockIdx.x; q += kBlock) before += w.part[q];
    uint64_t carry;
    block_scan_excl<kBlock, uint64_t>(before, tmp, &carry);
    for (int64_t r0 = b0; r0 < b1; r0 += kBlock) {  // uniform
        const int64_t i = r0 + threadIdx.x;
        const uint64_t v = i < b1 ? w.ebits[i] : 0;
        uint64_t t;
        const uint64_t x = block_scan_excl<kBlock, uint64_t>(v, tmp, &t);
        if (i < b1) w.eboff[i] = carry + x;
        carry += t;
    }
    const bool last = b0 < neb ? b1 == neb : (blockIdx.x == 0 && neb == 0);
    if (last && threadIdx.x == 0) w.eboff[neb] = carry;
}

// split: the flat prefix (eboff) is done already (k_enc_scan_part and
// k_enc_scan_apply); only the per-stream tables are left.
__global__ __launch_bounds__(1024) void k_enc_scan(int32_t S, int64_t word_cap, EncWs w,
                                                  uint64_t* __restrict__ word_off, uint64_t* __restrict__ nbits,
                                                  uint32_t* status, int32_t split)
{
    __shared__ uint64_t tmp[1024 / 64 + 1];
    constexpr int NW = 1024 / 64;
    const int64_t neb = split ? 0 : w.ebpre[S];  // split: the flat scan below does nothing
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t L = cdiv(cdiv(neb, (int64_t)NW), (int64_t)64) * 64;
    const int64_t b = min(wave * L, neb), e = min(b + L, neb);
    // clamped, unconditional loads, kEncScanU steps at a time
    auto load = [&](int64_t i0, uint64_t (&v)[kEncScanU]) {
#pragma unroll
        for (int u = 0; u < kEncScanU; ++u) {
            const int64_t i = i0 + u * 64 + lane;
            v[u] = w.ebits[min(i, e - 1)];
            if (i >= e) v[u] = 0;
        }
    };
    uint64_t local = 0;
    for (int64_t i0 = b; i0 < e; i0 += kEncScanU * 64) {
        uint64_t v[kEncScanU];
        load(i0, v);
#pragma unroll
        for (int u = 0; u < kEncScanU; ++u) local += v[u];
    }
    for (int d = 32; d >= 1; d >>= 1) local += __shfl_xor(local, d, 64);
    if (lane == 0) tmp[wave] = local;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint64_t run = 0;
        for (int i = 0; i < NW; ++i) { uint64_t q = tmp[i]; tmp[i] = run; run += q; }
        tmp[NW] = run;
    }
    __syncthreads();
    uint64_t carry = tmp[wave];
    for (int64_t i0 = b; i0 < e; i0 += kEncScanU * 64) {
        uint64_t v[kEncScanU];
        load(i0, v);
#pragma unroll
        for (int u = 0; u < kEncScanU; ++u) {
            uint64_t x = v[u];
            for (int d = 1; d < 64; d <<= 1) {
                const uint64_t y = __shfl_up(x, d, 64);
                if (lane >= d) x += y;
            }
            const int64_t i = i0 + u * 64 + lane;
            if (i < e) w.eboff[i] = carry + x - v[u];
            carry += __shfl(x, 63, 64);
        }
    }
    if (threadIdx.x == 0 && !split) w.eboff[neb] = tmp[NW];
    __syncthreads();
    // per stream, one thread each in rounds: first bit, word offset, bit count
    uint64_t words = 0;  // carried from round to round
    for (int64_t s0 = 0; s0 < S; s0 += 1024) {
        const int64_t s = s0 + threadIdx.x;
        const bool in = s < S;
        const uint64_t b0 = in ? w.eboff[w.ebpre[s]] : 0;
        const uint64_t nb = in ? w.eboff[w.ebpre[s + 1]] - b0 : 0;
        uint64_t tw;
        const uint64_t xw = words + block_scan_excl<1024, uint64_t>((nb + 31) / 32, tmp, &tw);
        if (in) {
            w.sbit0[s] = b0;
            word_off[s] = xw;
            nbits[s] = nb;
        }
        words += tw;
    }
    if (threadIdx.x != 0) return;
    word_off[S] = words;
    if (words > (uint64_t)word_cap) w.bad[0] |= 2u;  // only reachable with malformed input
    if (w.bad[0]) *status |= SGC_STATUS_BAD_INPUT;
}

constexpr int kEncLds = (int)kEncCodes + kEncAhead;
constexpr int kEncPer = (kEncLds + kBlock - 1) / kBlock;  // entries per thread in the LDS prefix
constexpr int kEncBufWords = 2048;  // LDS words a block assembles its output words in
static_assert(kEncBufWords % (4 * kBlock) == 0, "the word buffer is cleared in 16-byte stores");

typedef uint32_t u4e __attribute__((ext_vector_type(4)));

// OR v into buffer word k unless it is zero or not the block's.
__device__ inline void enc_or(uint32_t* buf, int64_t k, int32_t nbuf, uint32_t v)
{
    if (v && k >= 0 && k < nbuf) atomicOr(&buf[k], v);
}

// The code of gap z placed at aligned bit a: buffer word k holds aligned bits
// [32 (k + m0), 32 (k + m0) + 32).  A code of at most 33 bits is one shifted
// 64-bit pattern over two words; a longer one (long unary run) fills its
// words one by one, clamped to the block's words.  32-bit positions: a
// block's codes, look-ahead included, span less than 2^31 + 2080 * 31 bits
// (the gaps of a stream sum to less than 2^31), and a < that + 32.
__device__ inline void enc_put(uint32_t* buf, uint32_t a, uint32_t z, uint32_t b, int32_t m0, int32_t nbuf)
{
    const uint32_t q = z >> b;
    const uint64_t rem = z & ((1u << b) - 1u);
    const int64_t m = (int64_t)(a >> 5) - m0;
    if (q + 1 + b <= 33) {
        const uint64_t p = (((1ull << q) - 1ull) | (rem << (q + 1))) << (a & 31);
        enc_or(buf, m, nbuf, (uint32_t)p);
        enc_or(buf, m + 1, nbuf, (uint32_t)(p >> 32));
        return;
    }
    const uint32_t e = a + q;  // one-bits [a, e), the zero at e, the low bits after it
    const int32_t k0 = (int32_t)max(m, (int64_t)0), k1 = (int32_t)min((int64_t)((e - 1) >> 5) - m0, (int64_t)nbuf - 1);
    for (int32_t k = k0; k <= k1; ++k) {
        const uint32_t w0 = (uint32_t)(k + m0) * 32;
        const uint32_t lo = a > w0 ? a : w0, hi = e - w0 < 32 ? e : w0 + 32;
        const uint32_t nb = hi - lo;
        atomicOr(&buf[k], (nb >= 32 ? 0xffffffffu : ((1u << nb) - 1u)) << (lo - w0));
    }
    const uint64_t p = rem << ((e + 1) & 31);
    const int64_t mr = (int64_t)((e + 1) >> 5) - m0;
    enc_or(buf, mr, nbuf, (uint32_t)p);
    enc_or(buf, mr + 1, nbuf, (uint32_t)(p >> 32));
}

__global__ __launch_bounds__(kBlock) void k_enc_pack(const int32_t* __restrict__ idx, int32_t S, int32_t b, EncWs w,
                                                    uint32_t* __restrict__ words, const uint64_t* __restrict__ word_off,
                                                    uint64_t* __restrict__ chunk_off)
{
    __shared__ uint32_t zs[kEncLds];
    __shared__ uint32_t off[kEncLds + 1];
    __shared__ __align__(16) uint32_t buf[kEncBufWords];
    __shared__ uint32_t tmp[kBlock / 64 + 1];
    if (w.bad[0] & 2u) return;
    const int64_t neb = w.ebpre[S];
    for (int64_t blk = blockIdx.x; blk < neb; blk += gridDim.x) {
        const EncBlock k = enc_block(w, S, blk);
        const int nown = (int)(k.e1 - k.e0), ntot = nown + (int)k.ahead;
        // per-stream and per-block values, loaded before they are needed
        const EncStream st = enc_stream(w, k.s);
        const uint64_t B0 = w.eboff[blk] - w.sbit0[k.s];  // stream-relative first bit of the block
        const int64_t q0 = k.e0 - st.first;               // stream-relative index of the first code
        const int64_t chpre = w.chpre[k.s];
        uint32_t* sw = words + word_off[k.s];
        // the word buffer starts clear (the previous block's last barrier has passed)
#pragma unroll
        for (int q = 0; q < kEncBufWords / (4 * kBlock); ++q)
            *(u4e*)&buf[4 * (q * kBlock + threadIdx.x)] = u4e{0u, 0u, 0u, 0u};
        // gaps into LDS (coalesced, clamped, unconditional loads), then code
        // lengths thread-contiguous so that the prefix is one block scan
        {
            // pointers rebased to the block (uniform) and small unsigned
            // offsets: scalar base + 32-bit lane offset per load.  The entry
            // before code l is pb[l] inside a stream, and for a block that
            // starts its stream pb[max(l - 1, 0)] (code 0 has none)
            const int32_t* pc = idx + k.e0;
            const uint32_t sft = k.e0 > st.first ? 1u : 0u;
            const int32_t* pb = pc - sft;
            int32_t cur[kEncPer], bef[kEncPer];
#pragma unroll
            for (int q = 0; q < kEncPer; ++q) {
                const uint32_t l = (uint32_t)min(q * kBlock + (int)threadIdx.x, ntot - 1);
                cur[q] = pc[l];
                bef[q] = pb[sft ? l : (l ? l - 1 : 0u)];
            }
            bool bad = false;  // flagged by the length pass already
#pragma unroll
            for (int q = 0; q < kEncPer; ++q) {
                const int i = q * kBlock + threadIdx.x;
                if (i < ntot) zs[i] = enc_gap(cur[q], bef[q], st, k.e0 + i, &bad);
            }
        }
        __syncthreads();
        uint32_t zq[kEncPer], oq[kEncPer];
        uint32_t local = 0;
#pragma unroll
        for (int q = 0; q < kEncPer; ++q) {
            const int i = threadIdx.x * kEncPer + q;
            zq[q] = i < ntot ? zs[i] : 0u;
            oq[q] = local;
            local += i < ntot ? (zq[q] >> b) + 1 + (uint32_t)b : 0u;
        }
        uint32_t tot;
        const uint32_t run = block_exclusive_scan<uint32_t>(local, tmp, &tot);
#pragma unroll
        for (int q = 0; q < kEncPer; ++q) {
            const int i = threadIdx.x * kEncPer + q;
            oq[q] += run;
            if (i < ntot) off[i] = oq[q];
        }
        if (threadIdx.x == kBlock - 1) off[ntot] = tot;  // ntot <= kEncLds
        __syncthreads();
        const uint64_t B1 = B0 + off[nown];
        const uint64_t wfirst = (B0 + 31) / 32, wend = (B1 + 31) / 32;
        // The block writes every word whose first bit lies in it (the next
        // block's first codes complete the last one).  Usually each code ORs
        // its bits into those words in LDS and the words are stored once;
        // a block whose words exceed the buffer has each word assembled by
        // one thread from the codes that overlap it instead.
        if (wend - wfirst <= (uint64_t)kEncBufWords) {  // uniform
            const uint32_t h = (uint32_t)(B0 & 31);  // aligned bit 0 is stream bit B0 - h
            const int32_t m0 = h ? 1 : 0, nbuf = (int32_t)(wend - wfirst);
#pragma unroll
            for (int q = 0; q < kEncPer; ++q)
                if (threadIdx.x * kEncPer + q < ntot) enc_put(buf, oq[q] + h, zq[q], (uint32_t)b, m0, nbuf);
            __syncthreads();
            for (int32_t i = threadIdx.x; i < nbuf; i += kBlock) sw[wfirst + i] = buf[i];
        } else {
            for (uint64_t wd = wfirst + threadIdx.x; wd < wend; wd += kBlock) {
                const uint64_t W0 = wd * 32;
                // first code whose end lies past W0 (its start is <= W0 or it is code 0)
                int lo = 0, hi = ntot - 1;
                while (lo < hi) {
                    const int mid = (lo + hi) >> 1;
                    if (B0 + off[mid + 1] <= W0) lo = mid + 1; else hi = mid;
                }
                uint32_t v = 0;
                for (int i = lo; i < ntot; ++i) {
                    const uint64_t o = B0 + off[i];
                    if (o >= W0 + 32) break;
                    const uint32_t z = zs[i];
                    const uint64_t q = z >> b;
                    // unary one-bits [o, o+q)
                    const uint64_t a0 = o > W0 ? o : W0;
                    const uint64_t a1 = (o + q) < (W0 + 32) ? (o + q) : (W0 + 32);
                    if (a0 < a1) {
                        const uint32_t nbit = (uint32_t)(a1 - a0);
                        const uint32_t m = nbit >= 32 ? 0xffffffffu : ((1u << nbit) - 1u);
                        v |= m << (uint32_t)(a0 - W0);
                    }
                    // remainder bits start after the terminating zero
                    if (b > 0) {
                        const int64_t sh = (int64_t)(o + q + 1) - (int64_t)W0;
                        const uint64_t rem = (uint64_t)(z & ((1u << b) - 1u));
                        if (sh >= 0 && sh < 32) v |= (uint32_t)(rem << sh);
                        else if (sh < 0 && -sh < b) v |= (uint32_t)(rem >> (-sh));
                    }
                }
                sw[wd] = v;
            }
        }
        // chunk table: (bit offset, stream position reached before the code) of
        // every SGC_CHUNK_CODES-th code
        for (int i = threadIdx.x * SGC_CHUNK_CODES; i < nown; i += kBlock * SGC_CHUNK_CODES) {
            const int64_t c = chpre + (q0 + i) / SGC_CHUNK_CODES;
            const int64_t j = k.e0 + i;
            const int32_t before = idx[j > st.first ? j - 1 : j];  // unconditional load
            chunk_off[2 * c] = B0 + off[i];
            chunk_off[2 * c + 1] = j == st.first ? 0 : (uint64_t)((int64_t)before - st.base + 1);
        }
        __syncthreads();  // LDS reuse by the next block of this workgroup
    }
}

}  // namespace sgc

using namespace sgc;

extern "C" int64_t sgc_encode_word_bound(const sgc_layout* L, int32_t scope, int32_t b, int64_t cap)
{
    if (!L || (scope != SGC_GLOBAL && scope != SGC_PER_SEGMENT) || b < 0 || b > 30 || cap < 0) return -1;
    const int64_t bits = cap * (int64_t)(b + 1) + (L->n >> b);
    return cdiv(bits, 32) + enc_streams(L, scope);
}

extern "C" int64_t sgc_encode_chunk_bound(const sgc_layout* L, int32_t scope, int64_t cap)
{
    if (!L || (scope != SGC_GLOBAL && scope != SGC_PER_SEGMENT) || cap < 0) return -1;
    return 2 * (cdiv(cap, (int64_t)SGC_CHUNK_CODES) + enc_streams(L, scope));
}

extern "C" size_t sgc_encode_workspace(const sgc_layout* L, int32_t scope, int64_t cap)
{
    if (!L || (scope != SGC_GLOBAL && scope != SGC_PER_SEGMENT) || cap < 0) return 0;
    Carver c(nullptr);
    EncWs w;
    carve_enc(c, L, scope, cap, &w);
    return c.off;
}

extern "C" int sgc_encode(const sgc_layout* Lc, int32_t scope, int32_t b, const int32_t* idx, const int64_t* counts,
                          int64_t cap, uint32_t* out_words, int64_t word_cap, uint64_t* out_word_off,
                          uint64_t* out_nbits, uint64_t* out_chunk_off, int64_t chunk_cap, uint32_t* dstatus,
                          void* ws, size_t ws_bytes, sgc_stream_t stream)
{
    sgc_layout* L = const_cast<sgc_layout*>(Lc);
    if (!L || (scope != SGC_GLOBAL && scope != SGC_PER_SEGMENT) || b < 0 || b > 30) return SGC_EINVAL;
    if (cap < 0 || cap >= ((int64_t)1 << 31) || !counts || !out_word_off || !out_nbits) return SGC_EINVAL;
    if (cap > 0 && (!idx || !out_words || !out_chunk_off)) return SGC_EINVAL;
    if (word_cap < sgc_encode_word_bound(L, scope, b, cap)) return SGC_ENOSPC;
    if (chunk_cap < sgc_encode_chunk_bound(L, scope, cap)) return SGC_ENOSPC;
    Carver c0(nullptr);
    EncWs w0;
    carve_enc(c0, L, scope, cap, &w0);
    if (!ws || ws_bytes < c0.off) return SGC_ENOSPC;
    Carver c(ws);
    EncWs w;
    carve_enc(c, L, scope, cap, &w);
    DevTables* dt = nullptr;
    int rc = device_tables(L, &dt);
    if (rc) return rc;
    hipStream_t s = (hipStream_t)stream;
    const int32_t S = enc_streams(L, scope);
    uint32_t* status = dstatus ? dstatus : w.st;
    k_enc_setup<<<1, kBlock, 0, s>>>(counts, dt->seg_off, L->nseg, scope, cap, w);
    SGC_LAUNCH_CHECK();
    const unsigned gb = (unsigned)std::min<int64_t>(enc_neb_max(L, scope, cap), 4096);
    k_enc_len<<<gb, kBlock, 0, s>>>(idx, S, b, w);
    SGC_LAUNCH_CHECK();
    const int64_t nebm = enc_neb_max(L, scope, cap);
    const int32_t split = nebm > kScanSplit ? 1 : 0;
    if (split) {
        const unsigned pb = (unsigned)cdiv(nebm, kScanPart);
        k_enc_scan_part<<<pb, kBlock, 0, s>>>(S, w);
        SGC_LAUNCH_CHECK();
        k_enc_scan_apply<<<pb, kBlock, 0, s>>>(S, w);
        SGC_LAUNCH_CHECK();
    }
    k_enc_scan<<<1, 1024, 0, s>>>(S, word_cap, w, out_word_off, out_nbits, status, split);
    SGC_LAUNCH_CHECK();
    k_enc_pack<<<gb, kBlock, 0, s>>>(idx, S, b, w, out_words, out_word_off, out_chunk_off);
    SGC_LAUNCH_CHECK();
    return SGC_OK;
}
