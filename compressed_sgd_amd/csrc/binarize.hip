// binarize.hip -- sparse binarization / 2-bit quantization of kept values.
//
// [SBC] §II Sparse Binarization: after top-p selection by magnitude the
// positive and negative kept values of a tensor are each summarised by
// their mean; only the side whose mean is larger in absolute value stays
// nonzero and is sent as that single mean.  [SBC] appendix C: the mean is
// the unique least-squares single value of the side.  [SBC] §II Residual
// Accumulation: whatever is not sent stays in the residual.  [AH17]
// Abstract: dropping can be combined with quantization (2-bit ternary here).
//
// GPU design: per-chunk partial sums (count and double sum per sign, fixed
// in-block tree order), one block per segment reduces its chunks in a fixed
// order, one block decides sides / means and scans the chunk output offsets,
// then an apply kernel writes the message and the residual.
#include "sgc_common.h"

namespace sgc {

struct BinWs {
    int64_t* estart;   // [nseg+1] entry prefix per segment
    int64_t* cpre;     // [nseg+1] chunk prefix per segment
    uint32_t* ccp;     // [nch] positive count per chunk
    uint32_t* ccn;     // [nch] negative count per chunk
    double* csp;       // [nch] positive sum per chunk
    double* csn;       // [nch] |negative| sum per chunk
    int64_t* cout;     // [nch+1] output offset per chunk (SBC)
    float* mpos;       // [nseg]
    float* mneg;       // [nseg]
    int32_t* side;     // [nseg] +1, -1, 0
    int64_t* segcp;    // [nseg]
    int64_t* segcn;    // [nseg]
    double* segsp;     // [nseg]
    double* segsn;     // [nseg]
};

static int64_t bin_nch_max(const sgc_layout* L, int64_t cap) { return cdiv(cap, kChunk) + L->nseg + 1; }

static void carve_bin(Carver& c, const sgc_layout* L, int64_t cap, BinWs* w)
{
    const int64_t ns = L->nseg, nch = bin_nch_max(L, cap);
    w->estart = c.take<int64_t>(ns + 1);
    w->cpre = c.take<int64_t>(ns + 1);
    w->ccp = c.take<uint32_t>(nch);
    w->ccn = c.take<uint32_t>(nch);
    w->csp = c.take<double>(nch);
    w->csn = c.take<double>(nch);
    w->cout = c.take<int64_t>(nch + 1);
    w->mpos = c.take<float>(ns);
    w->mneg = c.take<float>(ns);
    w->side = c.take<int32_t>(ns);
    w->segcp = c.take<int64_t>(ns);
    w->segcn = c.take<int64_t>(ns);
    w->segsp = c.take<double>(ns);
    w->segsn = c.take<double>(ns);
}

// Entry and chunk prefixes, one thread per segment in rounds (workgroup
// scans).  Counts are clamped into [0, cap] so that a malformed count table
// can never move a read outside the inputs: entry prefix = min(cap, prefix of
// the clamped counts), the same as clamping each count to the room left.
__global__ __launch_bounds__(kBlock) void k_bin_setup(const int64_t* __restrict__ counts, int32_t nseg, int64_t cap,
                                                     BinWs w)
{
    __shared__ int64_t tmp[kBlock / 64 + 1];
    int64_t P = 0, C = 0;  // prefixes carried from round to round
    for (int64_t t0 = 0; t0 < nseg; t0 += kBlock) {
        const int64_t t = t0 + threadIdx.x;
        const bool in = t < nseg;
        int64_t c = in ? counts[t] : 0;
        c = c < 0 ? 0 : (c > cap ? cap : c);
        int64_t tp, tc;
        const int64_t xp = P + block_scan_excl<kBlock, int64_t>(c, tmp, &tp);
        const int64_t e0 = xp < cap ? xp : cap, e1 = xp + c < cap ? xp + c : cap;
        const int64_t xc = C + block_scan_excl<kBlock, int64_t>(cdiv(e1 - e0, kChunk), tmp, &tc);
        if (in) {
            w.estart[t] = e0;
            w.cpre[t] = xc;
        }
        P += tp;
        C += tc;
    }
    if (threadIdx.x == 0) {
        w.estart[nseg] = P < cap ? P : cap;
        w.cpre[nseg] = C;
    }
}

// Deterministic block sum (fixed shuffle tree, then waves in order).
template <typename T>
__device__ inline T block_sum(T v, T* tmp)
{
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) v += __shfl_down(v, d, 64);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) tmp[wave] = v;
    __syncthreads();
    T s = 0;
    if (threadIdx.x == 0)
        for (int i = 0; i < (int)(blockDim.x >> 6); ++i) s += tmp[i];
    __syncthreads();
    return s;  // valid in thread 0
}

__global__ __launch_bounds__(kBlock) void k_bin_sums(const float* __restrict__ val, int32_t nseg, BinWs w)
{
    __shared__ double dt[kBlock / 64];
    __shared__ uint32_t ut[kBlock / 64];
    const int64_t nch = w.cpre[nseg];
    for (int64_t c = blockIdx.x; c < nch; c += gridDim.x) {
        const int64_t t = find_bucket(w.cpre, (int64_t)nseg + 1, c);
        const int64_t base = w.estart[t] + (c - w.cpre[t]) * kChunk;
        const int64_t end = min(base + kChunk, w.estart[t + 1]);
        uint32_t cp = 0, cn = 0;
        double sp = 0.0, sn = 0.0;
        // entry j*kBlock + tid of the chunk: coalesced loads.  Clamped and
        // unconditional, so that all are in flight at once (a guarded load
        // would be waited for before the next is issued)
        const int64_t b = base + threadIdx.x;
        float vv[kPer];
#pragma unroll
        for (int j = 0; j < kPer; ++j) vv[j] = val[min(b + j * kBlock, end - 1)];
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            if (b + j * kBlock < end) {
                const float v = vv[j];
                if (v > 0.0f) { ++cp; sp += (double)v; }
                else if (v < 0.0f) { ++cn; sn += -(double)v; }
            }
        }
        cp = block_sum<uint32_t>(cp, ut);
        cn = block_sum<uint32_t>(cn, ut);
        sp = block_sum<double>(sp, dt);
        sn = block_sum<double>(sn, dt);
        if (threadIdx.x == 0) {
            w.ccp[c] = cp;
            w.ccn[c] = cn;
            w.csp[c] = sp;
            w.csn[c] = sn;
        }
    }
}

// One block per segment: reduce its chunk partials in a fixed order.
__global__ __launch_bounds__(kBlock) void k_bin_segsum(int32_t nseg, BinWs w)
{
    __shared__ double dt[kBlock / 64];
    __shared__ int64_t it[kBlock / 64];
    for (int64_t t = blockIdx.x; t < nseg; t += gridDim.x) {
        int64_t cp = 0, cn = 0;
        double sp = 0.0, sn = 0.0;
        for (int64_t c = w.cpre[t] + threadIdx.x; c < w.cpre[t + 1]; c += kBlock) {
            cp += w.ccp[c];
            cn += w.ccn[c];
            sp += w.csp[c];
            sn += w.csn[c];
        }
        cp = block_sum<int64_t>(cp, it);
        cn = block_sum<int64_t>(cn, it);
        sp = block_sum<double>(sp, dt);
        sn = block_sum<double>(sn, dt);
        if (threadIdx.x == 0) {
            w.segcp[t] = cp;
            w.segcn[t] = cn;
            w.segsp[t] = sp;
            w.segsn[t] = sn;
        }
    }
}

// Means, side choice (fp32 comparison, positive wins a tie), outputs and
// the SBC chunk output offsets.
__global__ __launch_bounds__(1024) void k_bin_resolve(int32_t nseg, int32_t mode, BinWs w,
                                                     int64_t* __restrict__ out_counts, float* __restrict__ out_means)
{
    __shared__ int64_t tmp[1024 / 64 + 1];
    int64_t sent = 0;  // this thread's share of the output total
    for (int64_t t = threadIdx.x; t < nseg; t += blockDim.x) {
        const int64_t cp = w.segcp[t], cn = w.segcn[t];
        const float mp = cp ? (float)(w.segsp[t] / (double)cp) : 0.0f;
        const float mn = cn ? (float)(w.segsn[t] / (double)cn) : 0.0f;
        w.mpos[t] = mp;
        w.mneg[t] = mn;
        int32_t side = 0;
        if (cp + cn > 0) side = (mp >= mn) ? 1 : -1;
        w.side[t] = side;
        if (mode == SGC_BIN_SBC) {
            out_means[t] = side > 0 ? mp : side < 0 ? -mn : 0.0f;
            out_counts[t] = side > 0 ? cp : side < 0 ? cn : 0;
            sent += side > 0 ? cp : side < 0 ? cn : 0;
        } else {
            out_means[2 * t] = mp;
            out_means[2 * t + 1] = -mn;
            out_counts[t] = w.estart[t + 1] - w.estart[t];
        }
    }
    int64_t total;
    block_scan_excl<1024, int64_t>(sent, tmp, &total);  // (also the barrier before w.side is read below)
    if (threadIdx.x == 0) out_counts[nseg] = mode == SGC_BIN_SBC ? total : w.estart[nseg];
    if (mode != SGC_BIN_SBC) return;
    // chunk output offsets: flat exclusive scan of the chosen count per chunk
    const int64_t nch = w.cpre[nseg];
    const int64_t per = cdiv(nch, (int64_t)blockDim.x);
    const int64_t b = threadIdx.x * per, e = min(b + per, nch);
    int64_t local = 0;
    for (int64_t c = b; c < e; ++c) {
        const int64_t t = find_bucket(w.cpre, (int64_t)nseg + 1, c);
        local += w.side[t] > 0 ? w.ccp[c] : w.side[t] < 0 ? w.ccn[c] : 0;
    }
    // block exclusive scan (1024 threads)
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int64_t x = local;
    for (int d = 1; d < 64; d <<= 1) {
        int64_t y = __shfl_up(x, d, 64);
        if (lane >= d) x += y;
    }
    if (lane == 63) tmp[wave] = x;
    __syncthreads();
    if (threadIdx.x == 0) {
        int64_t run = 0;
        for (int i = 0; i < (int)(blockDim.x >> 6); ++i) { int64_t q = tmp[i]; tmp[i] = run; run += q; }
    }
    __syncthreads();
    int64_t run = tmp[wave] + x - local;
    for (int64_t c = b; c < e; ++c) {
        w.cout[c] = run;
        const int64_t t = find_bucket(w.cpre, (int64_t)nseg + 1, c);
        run += w.side[t] > 0 ? w.ccp[c] : w.side[t] < 0 ? w.ccn[c] : 0;
    }
}

// held: the residual holds val at the kept entries already (only the sent
// side is written).  Entry j*kBlock + tid of a chunk belongs to thread tid
// (slot j): the loads are coalesced, and the 64 residual writes of one
// store instruction go to 64 consecutive kept entries, close together in
// memory.  Output offsets inside the chunk follow the entry order (slot,
// wave, lane): wave ballots give the lane prefix, LDS the wave totals.
__global__ __launch_bounds__(kBlock) void k_bin_apply_sbc(const int32_t* __restrict__ idx, const float* __restrict__ val,
                                                         int32_t nseg, BinWs w, float* __restrict__ res,
                                                         int64_t n, int32_t* __restrict__ out_idx, int64_t cap,
                                                         int32_t held)
{
    constexpr int NW = kBlock / 64;
    __shared__ uint32_t wcnt[kPer][NW];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
    const int64_t nch = w.cpre[nseg];
    for (int64_t c = blockIdx.x; c < nch; c += gridDim.x) {
        const int64_t t = find_bucket(w.cpre, (int64_t)nseg + 1, c);
        const int32_t side = w.side[t];
        const float mean = side > 0 ? w.mpos[t] : side < 0 ? -w.mneg[t] : 0.0f;
        const int64_t base = w.estart[t] + (c - w.cpre[t]) * kChunk;
        const int64_t end = min(base + kChunk, w.estart[t + 1]);
        // clamped, unconditional loads (see k_bin_sums)
        float vv[kPer];
        int32_t ii[kPer];
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int64_t i = min(base + j * kBlock + threadIdx.x, end - 1);
            vv[j] = val[i];
            ii[j] = idx[i];
        }
        uint32_t sel = 0, valid = 0;
        uint32_t pre[kPer];
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const bool in = base + j * kBlock + threadIdx.x < end;
            const float v = vv[j];
            const bool s = in && ((side > 0 && v > 0.0f) || (side < 0 && v < 0.0f));
            valid |= (uint32_t)in << j;
            sel |= (uint32_t)s << j;
            const uint64_t b = __ballot(s);
            pre[j] = (uint32_t)__popcll(b & below);
            if (lane == 0) wcnt[j][wave] = (uint32_t)__popcll(b);
        }
        __syncthreads();
        int64_t run = w.cout[c];
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            uint32_t before = 0, all = 0;
#pragma unroll
            for (int v = 0; v < NW; ++v) {
                const uint32_t q = wcnt[j][v];
                before += v < wave ? q : 0u;
                all += q;
            }
            const int64_t pos = run + before + pre[j];
            run += all;
            if (!((valid >> j) & 1u)) continue;
            const int32_t id = ii[j];
            if ((uint32_t)id >= (uint32_t)n) continue;
            if ((sel >> j) & 1u) {
                if (pos < cap) out_idx[pos] = id;
                res[id] = vv[j] - mean;
            } else if (!held) {
                res[id] = vv[j];
            }
        }
        __syncthreads();  // wcnt is rewritten by the next chunk
    }
}

// One lane per entry, 16 consecutive lanes per output word of 16 two-bit
// codes (their codes OR-ed together by shuffles): coalesced loads and
// stores, and every entry of the message in flight at once.  Each wave
// takes 4 words (64 entries) at a time; the segment of its first entry is
// found once and the lanes step forward over segment ends (rare).
__global__ __launch_bounds__(kBlock) void k_bin_apply_2bit(const int32_t* __restrict__ idx, const float* __restrict__ val,
                                                          int32_t nseg, BinWs w, float* __restrict__ res, int64_t n,
                                                          int32_t* __restrict__ out_idx, uint32_t* __restrict__ codes,
                                                          int32_t held)
{
    const int64_t total = w.estart[nseg];
    const int64_t nwords = cdiv(total, 16);
    const int lane = threadIdx.x & 63;
    const int64_t waves = (int64_t)gridDim.x * (kBlock / 64);
    for (int64_t w0 = ((int64_t)blockIdx.x * (kBlock / 64) + (threadIdx.x >> 6)) * 4; w0 < nwords; w0 += waves * 4) {
        const int64_t j0 = w0 * 16, j = j0 + lane;  // uniform per wave
        const bool in = j < total;
        const int64_t jc = in ? j : total - 1;  // clamped, unconditional loads
        const float v = val[jc];
        const int32_t id = idx[jc];
        int64_t t = find_bucket(w.estart, (int64_t)nseg + 1, j0);
        while (t + 1 < nseg && jc >= w.estart[t + 1]) ++t;  // a later segment (rare)
        const float mp = w.mpos[t], mn = w.mneg[t];
        const uint32_t code = !in ? 0u : v > 0.0f ? 1u : v < 0.0f ? 2u : 0u;
        const float qv = code == 1u ? mp : code == 2u ? -mn : 0.0f;
        // code 0: v - (+0) is v itself, already there when held
        if (in && (uint32_t)id < (uint32_t)n && (code != 0u || !held)) res[id] = v - qv;
        if (in && out_idx) out_idx[j] = id;
        uint32_t word = code << (2 * (lane & 15));
        for (int d = 1; d < 16; d <<= 1) word |= __shfl_xor(word, d, 64);
        const int64_t wd = w0 + (lane >> 4);
        if ((lane & 15) == 0 && wd < nwords) codes[wd] = word;
    }
}

}  // namespace sgc

using namespace sgc;

extern "C" size_t sgc_binarize_workspace(const sgc_layout* L, int64_t cap)
{
    if (!L || cap < 0) return 0;
    Carver c(nullptr);
    BinWs w;
    carve_bin(c, L, cap, &w);
    return c.off;
}

extern "C" int sgc_binarize(const sgc_layout* Lc, int32_t mode, const int32_t* idx, const float* val,
                            const int64_t* counts, int64_t cap, float* residual, int32_t* out_idx,
                            int64_t* out_counts, float* out_means, uint32_t* out_codes, void* ws, size_t ws_bytes,
                            sgc_stream_t stream)
{
    sgc_layout* L = const_cast<sgc_layout*>(Lc);
    const int32_t held = (mode & SGC_BIN_HELD) ? 1 : 0;
    mode &= ~(int32_t)SGC_BIN_HELD;
    if (!L || (mode != SGC_BIN_SBC && mode != SGC_BIN_2BIT)) return SGC_EINVAL;
    if (cap < 0 || cap >= ((int64_t)1 << 31)) return SGC_EINVAL;
    if (!counts || !out_counts || !out_means || (L->n > 0 && !residual)) return SGC_EINVAL;
    if (cap > 0 && (!idx || !val)) return SGC_EINVAL;
    if (mode == SGC_BIN_SBC && cap > 0 && !out_idx) return SGC_EINVAL;
    if (mode == SGC_BIN_2BIT && cap > 0 && !out_codes) return SGC_EINVAL;
    Carver c0(nullptr);
    BinWs w0;
    carve_bin(c0, L, cap, &w0);
    if (!ws || ws_bytes < c0.off) return SGC_ENOSPC;
    Carver c(ws);
    BinWs w;
    carve_bin(c, L, cap, &w);
    hipStream_t s = (hipStream_t)stream;
    const int32_t nseg = L->nseg;
    const int64_t nch_max = bin_nch_max(L, cap);
    const unsigned cb = (unsigned)std::min<int64_t>(nch_max, 2048);
    k_bin_setup<<<1, kBlock, 0, s>>>(counts, nseg, cap, w);
    SGC_LAUNCH_CHECK();
    k_bin_sums<<<cb, kBlock, 0, s>>>(val, nseg, w);
    SGC_LAUNCH_CHECK();
    k_bin_segsum<<<(unsigned)std::min<int64_t>(nseg, 1024), kBlock, 0, s>>>(nseg, w);
    SGC_LAUNCH_CHECK();
    k_bin_resolve<<<1, 1024, 0, s>>>(nseg, mode, w, out_counts, out_means);
    SGC_LAUNCH_CHECK();
    if (mode == SGC_BIN_SBC) {
        k_bin_apply_sbc<<<cb, kBlock, 0, s>>>(idx, val, nseg, w, residual, L->n, out_idx, cap, held);
    } else {
        const unsigned wb = (unsigned)std::max<int64_t>(1, std::min<int64_t>(cdiv(cap, kBlock), 4096));
        k_bin_apply_2bit<<<wb, kBlock, 0, s>>>(idx, val, nseg, w, residual, L->n, out_idx, out_codes, held);
    }
    SGC_LAUNCH_CHECK();
    return SGC_OK;
}
