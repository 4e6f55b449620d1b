// compress_gather.hip -- the gather pipeline of sgc_compress (selection
// over one ordered candidate array; the default at low kept fractions on
// vectors below 2^29 elements).
//
// Method ([SBC] §II Residual Accumulation and Sparse Binarization; [AH17]
// Abstract): acc = fp32(residual + grad); keep the largest-|acc| fraction
// of each selection group; send (index, value) ascending; the residual
// keeps everything else.
//
// GPU design (one HBM pass over the gradient in the common case):
//  1. probe   -- read a small sample of acc per group (runs of 16 elements)
//                and radix-select two bounds from it (top 21 key bits):
//                key_lo, a 6-sigma margin below the estimated k-th largest
//                magnitude key (the candidate bound), and key_z, the
//                estimate itself (the zeroing bound).  Sampled mode instead
//                takes the method's own systematic sample and its exact
//                threshold T, with key_lo = key_z = T.
//  2. pass 1  -- stream g and r once: acc = r + g; every element with
//                key >= key_lo goes into its tile's candidate region (wave
//                ballots + LDS offsets, index order kept); r is stored as
//                acc, or as +0 for key >= key_z, so that nearly all kept
//                entries leave the residual without a second, scattered
//                write.  A tile whose region overflows stores plain acc
//                everywhere.
//  3. scan    -- tile counts -> offsets (per 4096-tile super block, then
//                one small scan); per group: candidate count, and whether
//                the group is selected from its candidates or, if the probe
//                misled (fewer than k candidates) or the candidate array is
//                full, straight from the residual.
//  4. gather  -- one workgroup per 64 tiles copies their regions into one
//                ordered candidate array (sampled mode: into the output)
//                and counts the first radix digit of every candidate; an
//                overflowed tile is redone from r (= acc there).
//  5. select  -- exact k-th largest key per group over its candidates by a
//                3-digit radix select (11+10+10 bits, LDS histograms).
//  6. compact -- keep key > T, plus the first `quota` entries with key == T
//                in index order (lower index wins the tie); write idx/val
//                ascending; zero the residual only where pass 1 did not,
//                and give back acc to any entry pass 1 zeroed but the exact
//                selection did not keep.
#include "compress_path.h"

#include <cmath>

namespace sgc {
namespace gather {

typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int kSrcSamples = 0, kSrcCand = 1, kSrcDense = 2;
constexpr int kSuper = 4096;                     // tiles per scan super block
constexpr int kGatherTiles = 64;                 // tiles per gather workgroup (one wave lane each)
constexpr uint32_t kAccFlag = 0x80000000u;       // candidate index flag: r still holds acc there
constexpr int kRep = 8;                          // global histogram replicas per (virtual) group
constexpr int kHistBlocks = 1024;                // workgroups of a histogram pass
// The compaction's chunk-count scan runs in one workgroup unless the kept
// total exceeds kChunkSplit chunks' worth (kept fractions of ~10% and up at
// 2^30 elements); then it is split over workgroups of kChunkPart chunks.
constexpr int64_t kChunkPart = 4096;
constexpr int64_t kChunkSplit = 16384;

struct CompressWs {
    int64_t* k;        // [G] keep count
    int64_t* s;        // [G] probe / sample size
    int64_t* spre;     // [G+1] sample prefix
    int64_t* kpre;     // [G+1] keep-count prefix (exact output offsets)
    uint32_t* key_lo;  // [G] candidate bound
    uint32_t* key_z;   // [G] pass-1 zeroing bound
    // radix-select state, 2G virtual groups (probe: lower and upper bound)
    int32_t* src_kind; // [2G]
    int64_t* src_base; // [2G]
    int64_t* src_len;  // [2G]
    int64_t* rank;     // [2G] wanted rank (1-based); 0 = select nothing
    int64_t* cpre;     // [2G+1] chunk prefix over the selection source
    uint32_t* prefix;  // [2G] radix-select prefix -> T
    int64_t* mrem;     // [2G] remaining rank -> quota of ties at T
    uint32_t* hist;    // [2G * kRep * kBins] (kRep replicas spread the flush atomics)
    int64_t* cstart;   // [G] candidate array start per group
    float* samples;    // [S]
    uint32_t* tile_cnt;// [NT]
    int64_t* tile_loc; // [NT] exclusive prefix inside the super block
    int64_t* sup_pre;  // [NS+1] super block prefix
    int32_t* reg_idx;  // [NT * tcap]
    float* reg_val;    // [NT * tcap]
    float* reg_mom;    // [NT * tcap] u' of each candidate (momentum correction only)
    int32_t* cand_idx; // [capc]
    float* cand_val;   // [capc]
    float* cand_mom;   // [capc] (momentum correction only)
    uint32_t* ch_gt;   // [nch_max]
    uint32_t* ch_eq;   // [nch_max]
    int64_t* ch_gt_pre;// [nch_max+1]
    int64_t* ch_eq_pre;// [nch_max+1]
    int64_t* cpart;    // [2 * (nch_max / kChunkPart + 1)] (gt, eq) totals per part (split chunk scan)
    int64_t* scal;     // [8]: 0 output total, 1 candidate total
    uint32_t* status;  // [1] used when the caller passes no dstatus
    int32_t* over;     // [NT] tiles whose region overflowed (any order)
    uint32_t* nover;   // [1] entries in over
    uint32_t tcap;     // candidate slots per tile region (a power of two)
    uint32_t hold;     // SGC_HOLD_KEPT: kept entries keep acc in the residual (nothing is zeroed)
};

struct CompressSizes {
    int32_t G;
    int64_t NT, NS, S, capc, nch_max, tcap;
};

static CompressSizes compress_sizes(const sgc_layout* L, const sgc_compress_opts* o)
{
    CompressSizes z;
    std::vector<int64_t> off = host_group_off(L, o->scope);
    z.G = (int32_t)off.size() - 1;
    z.NT = (o->scope == SGC_GLOBAL) ? group_tiles(0, L->n) : L->seg_tile[L->nseg];
    z.NS = cdiv(z.NT, kSuper);
    z.tcap = region_capacity(o->keep_ppm);
    z.S = 0;
    int64_t K = 0;
    for (int32_t g = 0; g < z.G; ++g) {
        int64_t m = off[g + 1] - off[g];
        z.S += (o->mode == SGC_EXACT) ? probe_count(m) : sampled_count(m, o->sample_div, o->sample_min);
        K += keep_count(m, o->keep_ppm);
    }
    z.capc = (o->mode == SGC_EXACT) ? std::min<int64_t>(L->n, 4 * K + 262144) : 0;
    z.nch_max = cdiv(L->n + z.capc + 2 * z.S, kChunk) + 4 * (int64_t)z.G + 2;
    return z;
}

static void carve_compress(Carver& c, const CompressSizes& z, int mode, bool mom, CompressWs* w)
{
    const int64_t G = z.G, V = 2 * (int64_t)z.G;
    w->k = c.take<int64_t>(G);
    w->s = c.take<int64_t>(G);
    w->spre = c.take<int64_t>(G + 1);
    w->kpre = c.take<int64_t>(G + 1);
    w->key_lo = c.take<uint32_t>(G);
    w->key_z = c.take<uint32_t>(G);
    w->src_kind = c.take<int32_t>(V);
    w->src_base = c.take<int64_t>(V);
    w->src_len = c.take<int64_t>(V);
    w->rank = c.take<int64_t>(V);
    w->cpre = c.take<int64_t>(V + 1);
    w->prefix = c.take<uint32_t>(V);
    w->mrem = c.take<int64_t>(V);
    w->hist = c.take<uint32_t>(V * kRep * kBins);
    w->cstart = c.take<int64_t>(G);
    w->samples = c.take<float>(z.S);
    w->tile_cnt = c.take<uint32_t>(z.NT);
    w->tile_loc = c.take<int64_t>(z.NT);
    w->sup_pre = c.take<int64_t>(z.NS + 1);
    w->tcap = (uint32_t)z.tcap;
    w->reg_idx = c.take<int32_t>(z.NT * z.tcap);
    w->reg_val = c.take<float>(z.NT * z.tcap);
    w->reg_mom = mom ? c.take<float>(z.NT * z.tcap) : nullptr;
    w->cand_mom = nullptr;
    if (mode == SGC_EXACT) {
        w->cand_idx = c.take<int32_t>(z.capc);
        w->cand_val = c.take<float>(z.capc);
        if (mom) w->cand_mom = c.take<float>(z.capc);
        w->ch_gt = c.take<uint32_t>(z.nch_max);
        w->ch_eq = c.take<uint32_t>(z.nch_max);
        w->ch_gt_pre = c.take<int64_t>(z.nch_max + 1);
        w->ch_eq_pre = c.take<int64_t>(z.nch_max + 1);
        w->cpart = c.take<int64_t>(2 * (cdiv(z.nch_max, kChunkPart) + 1));
    } else {
        w->cand_idx = nullptr;
        w->cand_val = nullptr;
        w->ch_gt = w->ch_eq = nullptr;
        w->ch_gt_pre = w->ch_eq_pre = nullptr;
        w->cpart = nullptr;
    }
    w->scal = c.take<int64_t>(8);
    w->status = c.take<uint32_t>(1);
    w->over = c.take<int32_t>(z.NT);
    w->nover = c.take<uint32_t>(1);
}

// Global exclusive prefix of tile t (t == NT gives the total).
__device__ inline int64_t tile_prefix(const CompressWs& w, int64_t NT, int64_t t)
{
    return t >= NT ? w.sup_pre[cdiv(NT, kSuper)] : w.sup_pre[t / kSuper] + w.tile_loc[t];
}

// ----------------------------------------------------------------- setup
// Every thread clears the radix-select histograms (the resolve passes leave
// them clear again); workgroup 0 clears the library's own status word (when
// the caller passes none) and the overflow-list count, and goes over the
// groups in rounds of kBlock, one thread per group: keep counts, probe
// sizes, the two ranks (lower / upper bound) each group's probe selection
// needs, and their prefixes (workgroup scans).  counts_out (or NULL):
// exact mode with one segment per group -- the per-segment output counts
// are the groups' keep counts, written here.
__global__ __launch_bounds__(kBlock) void k_setup(const int64_t* __restrict__ goff, int32_t G, int32_t mode,
                                                 uint32_t ppm, uint32_t div, uint32_t smin, CompressWs w,
                                                 int64_t hist_words, uint32_t* clear_status,
                                                 int64_t* __restrict__ counts_out)
{
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < hist_words; i += (int64_t)gridDim.x * kBlock)
        w.hist[i] = 0;
    if (blockIdx.x != 0) return;
    if (threadIdx.x == 0) {
        if (clear_status) *clear_status = 0;
        *w.nover = 0;
    }
    __shared__ int64_t tmp[kBlock / 64 + 1];
    int64_t sp = 0, kp = 0, cp = 0;  // prefixes carried from round to round
    for (int64_t g0 = 0; g0 < G; g0 += kBlock) {
        const int64_t g = g0 + threadIdx.x;
        const bool in = g < G;
        int64_t k = 0, sz = 0, rlo = 0, rhi = 0;
        uint32_t klo = kNoKey, kz = kNoKey;
        if (in) {
            const int64_t m = goff[g + 1] - goff[g];
            k = keep_count(m, ppm);
            sz = (mode == SGC_EXACT) ? probe_count(m) : sampled_count(m, div, smin);
            if (mode == SGC_EXACT) {
                if (k > 0) {
                    if (sz == m) {
                        rlo = k;  // the probe read every element: its k-th key is the threshold
                        rhi = w.hold ? 0 : k;
                    } else {
                        // e: expected sampled keys above the true threshold.  The
                        // candidate bound takes a 6-sigma margin below it (a miss
                        // costs a dense selection); the zeroing bound sits at the
                        // estimate itself: either way it errs, the compaction
                        // fixes the few entries between it and the exact
                        // threshold with scattered writes
                        const double e = (double)sz * (double)k / (double)m;
                        const double d = 6.0 * sqrt(e) + 8.0;
                        const int64_t lo = (int64_t)(e + d) + 1;
                        const int64_t hi = (int64_t)(e + 0.5);
                        if (lo >= sz) klo = 0;  // the bound would be the sample minimum: take every element
                        else rlo = lo;
                        if (hi >= 1) rhi = hi;
                        if (w.hold) rhi = 0;  // no zeroing bound: nothing is zeroed
                    }
                }
            } else {
                rlo = keep_count(sz, ppm);  // the method's threshold; zeroing uses the same key
            }
        }
        const int64_t len0 = rlo > 0 ? sz : 0, len1 = rhi > 0 ? sz : 0;
        const int64_t c0 = cdiv(len0, kChunk), c1 = cdiv(len1, kChunk);
        int64_t ts, tk, tc;
        const int64_t xs = sp + block_scan_excl<kBlock, int64_t>(sz, tmp, &ts);
        const int64_t xk = kp + block_scan_excl<kBlock, int64_t>(k, tmp, &tk);
        const int64_t xc = cp + block_scan_excl<kBlock, int64_t>(c0 + c1, tmp, &tc);
        if (in) {
            w.k[g] = k;
            if (counts_out) counts_out[g] = k;
            w.s[g] = sz;
            w.spre[g] = xs;
            w.kpre[g] = xk;
            w.key_lo[g] = klo;
            w.key_z[g] = kz;
            for (int v = 0; v < 2; ++v) {
                const int64_t vg = 2 * g + v;
                const int64_t r = v == 0 ? rlo : rhi;
                w.rank[vg] = r;
                w.src_kind[vg] = kSrcSamples;
                w.src_base[vg] = xs;
                w.src_len[vg] = v == 0 ? len0 : len1;
                w.cpre[vg] = v == 0 ? xc : xc + c0;
                w.prefix[vg] = 0;
                w.mrem[vg] = r;
            }
        }
        sp += ts;
        kp += tk;
        cp += tc;
    }
    if (threadIdx.x == 0) {
        w.spre[G] = sp;
        w.kpre[G] = kp;
        w.cpre[2 * G] = cp;
        if (counts_out) counts_out[G] = kp;
    }
}

// Probe: acc = r + g (g replaced by u' = beta*u + g with momentum correction;
// u is only read here) at the sample positions.  Exact mode: runs of kRun
// contiguous elements at systematic unit positions (the whole group if it
// is small).  Sampled mode: the method's systematic single-element sample
// floor((2j+1) m / (2s)).
template <typename M>
__global__ __launch_bounds__(kBlock) void k_probe(const float* __restrict__ grad, const float* __restrict__ res,
                                                 const int64_t* __restrict__ goff, int32_t G, int32_t mode,
                                                 CompressWs w, int64_t S, M mom)
{
    for (int64_t j = (int64_t)blockIdx.x * kBlock + threadIdx.x; j < S; j += (int64_t)gridDim.x * kBlock) {
        const int64_t g = find_bucket(w.spre, (int64_t)G + 1, j);
        const int64_t m = goff[g + 1] - goff[g];
        const int64_t s = w.s[g];
        const uint64_t jj = (uint64_t)(j - w.spre[g]);
        int64_t pos;
        if (mode == SGC_EXACT) {
            const int64_t P = probe_points(m);
            if (P == 0) {
                pos = goff[g] + (int64_t)jj;
            } else {
                const uint64_t pt = jj / kRun, units = (uint64_t)(m / kRun);
                const uint64_t unit = ((2 * pt + 1) * units) / (2 * (uint64_t)P);
                pos = goff[g] + (int64_t)(unit * kRun + jj % kRun);
            }
        } else {
            pos = goff[g] + (int64_t)(((2 * jj + 1) * (uint64_t)m) / (2 * (uint64_t)s));
        }
        const float gp = M::on ? mom_update(mom.beta, mom.u[pos], grad[pos]) : grad[pos];
        w.samples[j] = res[pos] + gp;
    }
}

// ----------------------------------------------------------- radix select
// Histogram of one digit over every selection source chunk whose (virtual)
// group is still open and whose key matches the digits chosen so far.  Each
// workgroup takes a contiguous run of chunks and accumulates in LDS across
// them, flushing once per group it touches into one of kRep global replicas.
// Pick the digit holding the wanted rank (counted from the largest key) of
// virtual group g: sum the replicas, scan from the top, clear the replicas for
// the next digit.  Every thread of the block calls it (block scan inside).
// probe_last: this is the last digit of the probe selection; the resolving
// thread also stores the bound it yields (the chosen digits, low bits zero):
// even virtual groups give key_lo (and, in sampled mode, key_z = key_lo),
// odd ones key_z.
template <int D>
__device__ inline void resolve_group(const CompressWs& w, int64_t g, int64_t* tmp, bool probe_last, int32_t mode)
{
    constexpr int nb = D == 0 ? 2048 : 1024;
    constexpr int bits = D == 0 ? 11 : 10;
    constexpr int low = D == 0 ? 20 : D == 1 ? 10 : 0;  // key bits below this digit
    constexpr int per = nb / kBlock;
    const int64_t target = w.mrem[g];
    if (target == 0) return;  // uniform
    uint32_t* gh = w.hist + g * kRep * kBins;
    // thread t owns bins [nb - (t+1)*per, nb - t*per): thread 0 the largest keys
    const int top = nb - threadIdx.x * per;
    uint32_t cnt[per];
    int64_t local = 0;
#pragma unroll
    for (int i = 0; i < per; ++i) {
        uint32_t c = 0;
#pragma unroll
        for (int r = 0; r < kRep; ++r) {
            c += gh[r * kBins + top - 1 - i];
            gh[r * kBins + top - 1 - i] = 0;
        }
        cnt[i] = c;
        local += c;
    }
    int64_t total;
    const int64_t above = block_exclusive_scan<int64_t>(local, tmp, &total);
    if (above < target && above + local >= target) {
        int64_t run = above;
        for (int i = 0; i < per; ++i) {
            const int bin = top - 1 - i;
            if (run + cnt[i] >= target) {
                const uint32_t pre = (w.prefix[g] << bits) | (uint32_t)bin;
                w.prefix[g] = pre;
                w.mrem[g] = target - run;
                if (probe_last) {
                    const uint32_t key = pre << low;
                    if (g & 1) {
                        w.key_z[g >> 1] = key;
                    } else {
                        w.key_lo[g >> 1] = key;
                        if (mode != SGC_EXACT && !w.hold) w.key_z[g >> 1] = key;
                    }
                }
                break;
            }
            run += cnt[i];
        }
    }
}

// LDS histogram count of one item per hitting lane.  The lanes that share
// the first hitting lane's bin are counted with one atomic: in a narrow key
// band most lanes of a wave fall into one bin, and same-address LDS atomics
// serialise.
__device__ inline void lds_count(uint32_t* h, bool hit, uint32_t bin)
{
    const uint64_t m = __ballot(hit);
    if (m == 0) return;  // uniform
    const int first = __builtin_ctzll(m);
    const uint32_t b0 = __shfl(bin, first, 64);
    const bool same = hit && bin == b0;
    const uint64_t sm = __ballot(same);
    if ((int)(threadIdx.x & 63) == first) atomicAdd(&h[b0], (uint32_t)__popcll(sm));
    if (hit && !same) atomicAdd(&h[bin], 1u);
}

// Histogram of digit D over every virtual group's selection source, chunks
// split evenly over the workgroups; a chunk is kPer loads per thread, all in
// flight before the first is counted.  skip_cand: the digit of groups
// selected from their candidates was counted already (by the gather).
template <int D>
__global__ __launch_bounds__(kBlock) void k_srs_hist(const float* __restrict__ res, int32_t V, CompressWs w,
                                                    int32_t skip_cand)
{
    constexpr int shift = D == 0 ? 20 : D == 1 ? 10 : 0;
    constexpr uint32_t mask = D == 0 ? 0x7ffu : 0x3ffu;
    constexpr int nb = D == 0 ? 2048 : 1024;
    __shared__ uint32_t h[nb];
    const int64_t nch = w.cpre[V];
    const int64_t per = cdiv(nch, (int64_t)gridDim.x);
    const int64_t c0 = (int64_t)blockIdx.x * per, c1 = min(c0 + per, nch);
    if (c0 >= c1) return;  // uniform
    for (int b = threadIdx.x; b < nb; b += kBlock) h[b] = 0;
    __syncthreads();
    int64_t cur = -1;
    bool dirty = false;
    auto flush = [&](int64_t g) {
        __syncthreads();
        uint32_t* gh = w.hist + (g * kRep + (blockIdx.x & (kRep - 1))) * kBins;
        for (int b = threadIdx.x; b < nb; b += kBlock) {
            const uint32_t v = h[b];
            if (v) {
                atomicAdd(&gh[b], v);
                h[b] = 0;
            }
        }
        __syncthreads();
    };
    for (int64_t c = c0; c < c1; ++c) {
        const int64_t g = find_bucket(w.cpre, (int64_t)V + 1, c);  // uniform
        if (g != cur) {
            if (dirty) flush(cur);
            cur = g;
            dirty = false;
        }
        const int kind = w.src_kind[g];
        if (w.mrem[g] == 0 || (skip_cand && kind == kSrcCand)) continue;
        dirty = true;
        const int64_t base = w.src_base[g] + (c - w.cpre[g]) * kChunk;
        const int64_t end = min(base + kChunk, w.src_base[g] + w.src_len[g]);
        const float* src = kind == kSrcSamples ? w.samples : kind == kSrcCand ? w.cand_val : res;
        const uint32_t pre = w.prefix[g];
        // clamped, unconditional loads: a guarded load would be waited for
        // before the next one is issued
        float x[kPer];
#pragma unroll
        for (int j = 0; j < kPer; ++j) x[j] = src[min(base + j * kBlock + threadIdx.x, end - 1)];
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const uint32_t key = mag_key(x[j]);
            const bool hit = base + j * kBlock + threadIdx.x < end && (D == 0 || (key >> (shift + 10)) == pre);
            lds_count(h, hit, (key >> shift) & mask);
        }
    }
    if (dirty) flush(cur);
}

template <int D>
__global__ __launch_bounds__(kBlock) void k_srs_resolve(CompressWs w, int32_t probe_last, int32_t mode)
{
    __shared__ int64_t tmp[kBlock / 64 + 1];
    resolve_group<D>(w, blockIdx.x, tmp, probe_last != 0, mode);
}

// ---------------------------------------------------------------- pass 1
// Candidates of one tile in index order through `sink(pos, i, v, u')`, for a
// workgroup of TB threads holding SL float4 slots each (TB * SL * 4 =
// kTile).  ADD: acc = r + g is formed and r is stored (acc, or +0 for key >=
// kz when the tile's candidates fit its tcap-slot region); otherwise r already holds acc
// (redo of an overflowed tile).  With momentum correction g is replaced by
// u' = beta*u + g, and u is stored like r (u', or +0 where r gets +0); a redo
// reads u' back from u.  Returns the tile's candidate count to every
// thread.  Indices are 32-bit (n < 2^31); the tile base is uniform, so each
// access is a scalar base plus one 32-bit lane offset.  A tile that lies
// entirely inside its group skips every per-element range check.
template <bool ADD, int TB, int SL, typename M, typename Sink>
__device__ inline uint32_t tile_candidates(const float* __restrict__ grad, float* __restrict__ res, int32_t lo,
                                           int32_t hi, int32_t A, uint32_t klo, uint32_t kz, uint32_t tcap, M m,
                                           Sink sink)
{
    static_assert((int64_t)TB * SL * 4 == kTile, "a tile is TB threads x SL float4");
    constexpr int NW = TB / 64;
    __shared__ uint32_t wtot[SL][NW];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const bool full = A >= lo && (int64_t)A + kTile <= (int64_t)hi;  // uniform; 64-bit: A + kTile may reach 2^31
    const f4* rb = (const f4*)(res + A);
    const f4* gb = (const f4*)(grad + A);
    const f4* ub = M::on ? (const f4*)(m.u + A) : nullptr;  // momentum correction only
    f4 acc[SL];
    f4 um[SL];  // u' (momentum correction only; r or u already hold acc / u' when !ADD)
    if (full) {
#pragma unroll
        for (int u = 0; u < SL; ++u) {
            const int o = u * TB + tid;
            if (ADD) {
                const f4 rv = __builtin_nontemporal_load(rb + o);
                f4 gv = __builtin_nontemporal_load(gb + o);
                if constexpr (M::on) {
                    const f4 uo = __builtin_nontemporal_load(ub + o);
#pragma unroll
                    for (int j = 0; j < 4; ++j) gv[j] = mom_update(m.beta, uo[j], gv[j]);
                    um[u] = gv;
                }
                acc[u] = rv + gv;
            } else {
                acc[u] = rb[o];
                if constexpr (M::on) um[u] = ub[o];
            }
        }
    } else {
#pragma unroll
        for (int u = 0; u < SL; ++u) {
            const int32_t e = A + 4 * (u * TB + tid);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float a = 0.0f, up = 0.0f;
                if (e + j >= lo && e + j < hi) {
                    if (ADD) {
                        float gv = grad[e + j];
                        if constexpr (M::on) gv = mom_update(m.beta, m.u[e + j], gv);
                        up = gv;
                        a = res[e + j] + gv;
                    } else {
                        a = res[e + j];
                        if constexpr (M::on) up = m.u[e + j];
                    }
                }
                acc[u][j] = a;
                if constexpr (M::on) um[u][j] = up;
            }
        }
    }
    uint32_t flags = 0;  // 4 bits per slot
    uint32_t pre[SL];
#pragma unroll
    for (int u = 0; u < SL; ++u) {
        const int32_t e = A + 4 * (u * TB + tid);
        uint32_t f = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if ((full || (e + j >= lo && e + j < hi)) && mag_key(acc[u][j]) >= klo) f |= 1u << j;
        flags |= f << (4 * u);
        const uint32_t cnt = __popc(f);
        const uint64_t b0 = __ballot(cnt & 1u), b1 = __ballot(cnt & 2u), b2 = __ballot(cnt & 4u);
        const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
        pre[u] = __popcll(b0 & below) + 2u * __popcll(b1 & below) + 4u * __popcll(b2 & below);
        if (lane == 0) wtot[u][wave] = __popcll(b0) + 2u * __popcll(b1) + 4u * __popcll(b2);
    }
    __syncthreads();
    // offset of this lane's first candidate in slot u: every candidate of the
    // earlier slots, then of the earlier waves in slot u, then the wave prefix
    uint32_t run = 0;
#pragma unroll
    for (int u = 0; u < SL; ++u) {
        const uint32_t slot_base = run;
        uint32_t before = 0;
#pragma unroll
        for (int v = 0; v < NW; ++v) {
            const uint32_t c = wtot[u][v];
            before += v < wave ? c : 0u;
            run += c;
        }
        pre[u] += slot_base + before;
    }
    __syncthreads();  // wtot is reused by the next call in this block
    if (ADD) {
        const uint32_t z = run <= tcap ? kz : kNoKey;  // overflow: keep acc everywhere
        f4* rw = (f4*)(res + A);
        f4* uw = M::on ? (f4*)(m.u + A) : nullptr;
        if (full) {
#pragma unroll
            for (int u = 0; u < SL; ++u) {
                f4 st = acc[u], su;
                if constexpr (M::on) su = um[u];
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (mag_key(st[j]) >= z) {
                        st[j] = 0.0f;
                        if constexpr (M::on) su[j] = 0.0f;  // momentum masking
                    }
                __builtin_nontemporal_store(st, rw + u * TB + tid);
                if constexpr (M::on) __builtin_nontemporal_store(su, uw + u * TB + tid);
            }
        } else {
#pragma unroll
            for (int u = 0; u < SL; ++u) {
                const int32_t e = A + 4 * (u * TB + tid);
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (e + j >= lo && e + j < hi) {
                        const bool zero = mag_key(acc[u][j]) >= z;
                        res[e + j] = zero ? 0.0f : acc[u][j];
                        if constexpr (M::on) m.u[e + j] = zero ? 0.0f : um[u][j];
                    }
            }
        }
    }
    if (flags) {
#pragma unroll
        for (int u = 0; u < SL; ++u) {
            const uint32_t f = (flags >> (4 * u)) & 15u;
            if (!f) continue;
            const int32_t e = A + 4 * (u * TB + tid);
            uint32_t pos = pre[u];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (f & (1u << j)) sink(pos++, e + j, acc[u][j], M::on ? um[u][j] : 0.0f);
        }
    }
    return run;
}

__device__ inline int64_t tile_group(const int64_t* gtile, int32_t G, int64_t t)
{
    return G == 1 ? 0 : find_bucket(gtile, (int64_t)G + 1, t);
}

template <typename M>
__global__ __launch_bounds__(kPassThreads) void k_pass1(const float* __restrict__ grad, float* __restrict__ res,
                                                 const int64_t* __restrict__ goff, const int64_t* __restrict__ gtile,
                                                 int32_t G, CompressWs w, M m)
{
    const int64_t t = blockIdx.x;
    const int64_t g = tile_group(gtile, G, t);
    const int32_t lo = (int32_t)goff[g], hi = (int32_t)goff[g + 1];
    const int32_t A = (lo & ~3) + (int32_t)(t - gtile[g]) * (int32_t)kTile;
    int32_t* ridx = w.reg_idx + t * w.tcap;
    float* rval = w.reg_val + t * w.tcap;
    float* rmom = M::on ? w.reg_mom + t * w.tcap : nullptr;
    const uint32_t cnt = tile_candidates<true, kPassThreads, (int)(kTile / (4 * kPassThreads))>(
        grad, res, lo, hi, A, w.key_lo[g], w.key_z[g], w.tcap, m, [&](uint32_t pos, int32_t i, float v, float up) {
            if (pos < w.tcap) {
                ridx[pos] = i;
                rval[pos] = v;
                if constexpr (M::on) rmom[pos] = up;
            }
        });
    if (threadIdx.x == 0) w.tile_cnt[t] = cnt;
}

// ----------------------------------------------------------------- scans
constexpr int kScanThreads = 1024;

template <typename T>
__device__ inline T block1024_exclusive_scan(T v, T* tmp /*17*/, T* total)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    T x = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        T y = __shfl_up(x, d, 64);
        if (lane >= d) x += y;
    }
    if (lane == 63) tmp[wave] = x;
    __syncthreads();
    if (threadIdx.x == 0) {
        T run = 0;
        for (int i = 0; i < kScanThreads / 64; ++i) { T t = tmp[i]; tmp[i] = run; run += t; }
        tmp[kScanThreads / 64] = run;
    }
    __syncthreads();
    T res = tmp[wave] + x - v;
    *total = tmp[kScanThreads / 64];
    __syncthreads();
    return res;
}

// Exclusive prefix (int64) of `count` uint32 values, one block of 1024
// threads each owning a contiguous run.
__device__ inline void scan_u32_to_i64(const uint32_t* in, int64_t* out, int64_t count)
{
    __shared__ int64_t tmp[kScanThreads / 64 + 1];
    const int64_t per = cdiv(count, kScanThreads);
    const int64_t b = threadIdx.x * per, e = min(b + per, count);
    int64_t local = 0;
    int64_t i = b;
    for (; i + 8 <= e; i += 8) {  // eight independent loads in flight
        uint32_t v[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) v[q] = in[i + q];
#pragma unroll
        for (int q = 0; q < 8; ++q) local += v[q];
    }
    for (; i < e; ++i) local += in[i];
    int64_t total;
    int64_t run = block1024_exclusive_scan<int64_t>(local, tmp, &total);
    for (i = b; i + 8 <= e; i += 8) {
        uint32_t v[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) v[q] = in[i + q];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            out[i + q] = run;
            run += v[q];
        }
    }
    for (; i < e; ++i) {
        out[i] = run;
        run += in[i];
    }
    if (threadIdx.x == 0) out[count] = total;
    __syncthreads();
}

// Tile prefix inside each super block of kSuper tiles (16 per thread).
__global__ __launch_bounds__(kBlock) void k_tile_scan1(int64_t NT, CompressWs w)
{
    __shared__ int64_t tmp[kBlock / 64 + 1];
    constexpr int per = kSuper / kBlock;
    const int64_t t0 = (int64_t)blockIdx.x * kSuper + threadIdx.x * per;
    uint32_t c[per];
    int64_t local = 0;
#pragma unroll
    for (int q = 0; q < per; ++q) {
        c[q] = t0 + q < NT ? w.tile_cnt[t0 + q] : 0u;
        local += c[q];
    }
    int64_t total;
    int64_t run = block_exclusive_scan<int64_t>(local, tmp, &total);
#pragma unroll
    for (int q = 0; q < per; ++q) {
        if (t0 + q < NT) w.tile_loc[t0 + q] = run;
        run += c[q];
        // a tile whose region overflowed is redone by the gather, from this list
        if (c[q] > w.tcap) w.over[atomicAdd(w.nover, 1u)] = (int32_t)(t0 + q);
    }
    if (threadIdx.x == 0) w.sup_pre[blockIdx.x] = total;  // block sum; k_tile_scan2 makes it a prefix
}

// Super block prefix, then per group: candidate count, source of the main
// selection (candidates, or the dense residual), and chunk prefix.
__global__ __launch_bounds__(kScanThreads) void k_tile_scan2(const int64_t* __restrict__ goff,
                                                            const int64_t* __restrict__ gtile, int32_t G, int64_t NT,
                                                            int32_t mode, int64_t capc, int64_t cap, CompressWs w,
                                                            uint32_t* status)
{
    __shared__ int64_t tmp[kScanThreads / 64 + 1];
    const int64_t NS = cdiv(NT, kSuper);
    // exclusive scan of the NS block sums in place (NS is at most a few hundred)
    const int64_t per = cdiv(NS, kScanThreads);
    const int64_t b = threadIdx.x * per, e = min(b + per, NS);
    int64_t local = 0;
    for (int64_t i = b; i < e; ++i) local += w.sup_pre[i];
    int64_t total;
    int64_t run = block1024_exclusive_scan<int64_t>(local, tmp, &total);
    for (int64_t i = b; i < e; ++i) {
        const int64_t v = w.sup_pre[i];
        w.sup_pre[i] = run;
        run += v;
    }
    if (threadIdx.x == 0) {
        w.sup_pre[NS] = total;
        w.scal[1] = total;
        if (mode == SGC_SAMPLED) {
            w.scal[0] = total < cap ? total : cap;
            if (total > cap) *status |= SGC_STATUS_TRUNCATED;
        }
    }
    __syncthreads();  // every block prefix, the total included, is visible to the whole workgroup
    if (mode == SGC_SAMPLED) return;  // uniform
    // Per group, one thread each, in rounds: a group is selected from its
    // candidates when it has at least k of them and they fit the candidate
    // array after those of every earlier group that has at least its k
    // (a group that does not fit leaves a hole: nothing reads it); otherwise
    // straight from the residual.  Either way gives the same result.
    int64_t used = 0, cp = 0;  // prefixes carried from round to round
    bool dense = false;
    for (int64_t g0 = 0; g0 < G; g0 += kScanThreads) {
        const int64_t g = g0 + threadIdx.x;
        const bool in = g < G;
        int64_t cg = 0, k = 0;
        if (in) {
            cg = tile_prefix(w, NT, gtile[g + 1]) - tile_prefix(w, NT, gtile[g]);
            k = w.k[g];
        }
        const bool elig = in && k > 0 && cg >= k;
        int64_t tu;
        const int64_t xu = used + block1024_exclusive_scan<int64_t>(elig ? cg : 0, tmp, &tu);
        int kind = kSrcCand;
        int64_t base = xu, len = 0;
        if (in && k > 0) {
            if (elig && xu + cg <= capc) {
                len = cg;
            } else {
                kind = kSrcDense;
                base = goff[g];
                len = goff[g + 1] - goff[g];
                dense = true;
            }
        }
        int64_t tc;
        const int64_t xc = cp + block1024_exclusive_scan<int64_t>(in ? cdiv(len, kChunk) : 0, tmp, &tc);
        if (in) {
            w.cstart[g] = base;
            w.src_kind[g] = kind;
            w.src_base[g] = base;
            w.src_len[g] = len;
            w.rank[g] = k;
            w.prefix[g] = 0;
            w.mrem[g] = k;
            w.cpre[g] = xc;
        }
        used += tu;
        cp += tc;
    }
    dense = __syncthreads_or(dense);
    if (threadIdx.x != 0) return;
    w.cpre[G] = cp;
    w.scal[0] = w.kpre[G];
    if (dense) *status |= SGC_STATUS_DENSE_PATH;
}

// ----------------------------------------------------------------- gather
// One workgroup per kGatherTiles tiles.  Exact mode: copy the regions of
// candidate-selected groups into the ordered candidate array (indices of
// redone, overflowed tiles carry kAccFlag: pass 1 did not zero them) and
// count the first radix digit of every copied candidate -- in LDS for the
// group of the workgroup's first tile, straight into the global histogram
// for any other; for groups that fall back to the dense residual, give back
// acc to the entries pass 1 zeroed.  Sampled mode: the candidates are the
// output; entries beyond cap get their acc back (they stay in the residual).
// With momentum correction u' travels with each candidate and is given back
// to u wherever acc is given back to r; a redone entry that is sent has its
// momentum zeroed here (sampled) or in the compaction (exact).
constexpr int kGatherPer = 8;  // region entries per thread per round, loads all in flight
constexpr uint32_t kWaveGatherCap = 1024;  // regions this large (or larger) are copied a tile per wave

template <typename M>
__global__ __launch_bounds__(kBlock) void k_gather(const float* __restrict__ grad, float* __restrict__ res,
                                                  const int64_t* __restrict__ goff, const int64_t* __restrict__ gtile,
                                                  int32_t G, int64_t NT, int32_t mode,
                                                  int32_t* __restrict__ out_idx, float* __restrict__ out_val,
                                                  int64_t cap, CompressWs w, M m)
{
    __shared__ int64_t s_dst[kGatherTiles];   // destination of the tile's first entry (-1: restore only)
    __shared__ uint32_t s_pre[kGatherTiles + 1];  // prefix of the entries copied from the regions
    __shared__ uint32_t s_z[kGatherTiles];    // zeroing bound of the tile's group
    __shared__ int32_t s_hg[kGatherTiles];    // group whose first digit the tile counts (-1: none)
    __shared__ uint32_t h[kBins];             // first-digit histogram of group s_hg[0]
    static_assert(kGatherTiles == 64, "one wave lane per tile");
    const bool sampled = mode == SGC_SAMPLED;
    const int64_t t0 = (int64_t)blockIdx.x * kGatherTiles;
    if (!sampled)
        for (int b = threadIdx.x; b < kBins; b += kBlock) h[b] = 0;
    if (threadIdx.x < 64) {
        const int q = threadIdx.x;
        const int64_t t = t0 + q;
        int64_t dst = -1;
        uint32_t c = 0, z = kNoKey;
        int32_t hg = -1;
        bool over = false;
        if (t < NT) {
            const int64_t g = tile_group(gtile, G, t);
            c = w.tile_cnt[t];
            over = c > w.tcap;
            z = w.key_z[g];
            if (sampled) {
                dst = tile_prefix(w, NT, t);
            } else if (w.src_kind[g] == kSrcCand) {
                dst = w.cstart[g] + tile_prefix(w, NT, t) - tile_prefix(w, NT, gtile[g]);
                if (w.rank[g] > 0) hg = (int32_t)g;
            }
            if (over) c = 0;
        }
        s_dst[q] = dst;
        s_z[q] = z;
        s_hg[q] = hg;
        uint32_t x = c;  // inclusive scan over the wave
        for (int d = 1; d < 64; d <<= 1) {
            const uint32_t y = __shfl_up(x, d, 64);
            if (q >= d) x += y;
        }
        s_pre[q + 1] = x;
        if (q == 0) s_pre[0] = 0;
    }
    __syncthreads();
    const int32_t g_lds = s_hg[0];
    uint32_t* const ghist = w.hist + (blockIdx.x & (kRep - 1)) * kBins;  // + group * kRep * kBins
    // entry j of tile q (value v, index i, u' um) where it belongs: the
    // candidate array (counting its first digit), the output (sampled), or
    // back into the residual (dense-path groups); every lane of the wave
    // calls it (the digit count takes wave ballots), ok = the entry exists
    auto place = [&](int q, uint32_t j, int32_t i, float v, float um, bool ok) {
        const uint32_t bin = mag_key(v) >> 20;
        bool lds_hit = false;
        if (ok) {
            const int64_t dst = s_dst[q];
            if (dst < 0) {  // dense-path group: undo pass-1 zeroing
                if (mag_key(v) >= s_z[q]) {
                    res[i] = v;
                    if constexpr (M::on) m.u[i] = um;
                }
            } else if (sampled) {
                const int64_t p = dst + j;
                if (p < cap) {
                    out_idx[p] = i;
                    out_val[p] = v;
                } else {
                    res[i] = v;  // truncated: stays in the residual (and keeps its momentum)
                    if constexpr (M::on) m.u[i] = um;
                }
            } else {
                w.cand_idx[dst + j] = i;
                w.cand_val[dst + j] = v;
                if constexpr (M::on) w.cand_mom[dst + j] = um;
                const int32_t hg = s_hg[q];
                if (hg >= 0 && hg == g_lds) lds_hit = true;
                else if (hg >= 0) atomicAdd(&ghist[(int64_t)hg * kRep * kBins + bin], 1u);
            }
        }
        if (!sampled) lds_count(h, lds_hit, bin);
    };
    if (w.tcap >= kWaveGatherCap) {  // uniform
        // full regions (high kept fractions): each wave copies whole tiles, 64
        // consecutive entries per load -- no search for the tile of an entry
        const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
        for (int q = wave; q < kGatherTiles; q += kBlock / 64) {
            const uint32_t c = s_pre[q + 1] - s_pre[q];  // 0 for an overflowed tile (redone below)
            const int64_t rb = (t0 + q) * w.tcap;
            for (uint32_t j0 = 0; j0 < c; j0 += 64 * kGatherPer) {  // uniform per wave
                int32_t id[kGatherPer];
                float v[kGatherPer], um[kGatherPer];
#pragma unroll
                for (int u = 0; u < kGatherPer; ++u) {  // clamped, unconditional loads (all in flight)
                    const int64_t at = rb + min(j0 + u * 64 + lane, c - 1);
                    id[u] = w.reg_idx[at];
                    v[u] = w.reg_val[at];
                    um[u] = M::on ? w.reg_mom[at] : 0.0f;
                }
#pragma unroll
                for (int u = 0; u < kGatherPer; ++u) {
                    const uint32_t j = j0 + u * 64 + lane;
                    place(q, j, id[u], v[u], um[u], j < c);
                }
            }
        }
    } else {
        const uint32_t E = s_pre[kGatherTiles];
        for (uint32_t e0 = 0; e0 < E; e0 += kBlock * kGatherPer) {  // uniform
            int32_t id[kGatherPer];
            float v[kGatherPer], um[kGatherPer];
            int qs[kGatherPer];
#pragma unroll
            for (int u = 0; u < kGatherPer; ++u) {  // clamped, unconditional loads (all in flight)
                const uint32_t e = min(e0 + u * kBlock + threadIdx.x, E - 1);
                int q = 0;  // last tile whose entries start at or before e
                for (int hb = 32; hb >= 1; hb >>= 1)
                    if (e >= s_pre[q + hb]) q += hb;
                const int64_t at = (t0 + q) * w.tcap + (e - s_pre[q]);
                id[u] = w.reg_idx[at];
                v[u] = w.reg_val[at];
                um[u] = M::on ? w.reg_mom[at] : 0.0f;
                qs[u] = e0 + u * kBlock + threadIdx.x < E ? q : -1;
            }
#pragma unroll
            for (int u = 0; u < kGatherPer; ++u) {
                const int q = qs[u] < 0 ? 0 : qs[u];
                place(q, e0 + u * kBlock + threadIdx.x - s_pre[q], id[u], v[u], um[u], qs[u] >= 0);
            }
        }
    }
    // overflowed tiles: redo from r (which pass 1 left as acc there).  The
    // tile scan listed them; every workgroup takes its share of the list, so
    // that clustered inputs (many overflowed tiles side by side) spread the
    // redo over the whole grid instead of a few workgroups.
    const uint32_t nover = *w.nover;
    for (uint32_t j = blockIdx.x; j < nover; j += gridDim.x) {  // uniform per block
        const int64_t t = w.over[j];
        const int64_t g = tile_group(gtile, G, t);
        int64_t dst;
        int32_t hg = -1;
        if (sampled) {
            dst = tile_prefix(w, NT, t);
        } else if (w.src_kind[g] == kSrcCand) {
            dst = w.cstart[g] + tile_prefix(w, NT, t) - tile_prefix(w, NT, gtile[g]);
            if (w.rank[g] > 0) hg = (int32_t)g;
        } else {
            continue;  // dense-path group: pass 1 left acc everywhere in this tile
        }
        const int32_t lo = (int32_t)goff[g], hi = (int32_t)goff[g + 1];
        const int32_t A = (lo & ~3) + (int32_t)(t - gtile[g]) * (int32_t)kTile;
        tile_candidates<false, kBlock, (int)(kTile / (4 * kBlock))>(grad, res, lo, hi, A, w.key_lo[g], kNoKey, w.tcap, m,
                                                                  [&](uint32_t pos, int32_t i, float v, float up) {
            const int64_t p = dst + pos;
            if (sampled) {
                if (p < cap) {
                    out_idx[p] = i;
                    out_val[p] = v;
                    if (!w.hold) res[i] = 0.0f;
                    if constexpr (M::on) m.u[i] = 0.0f;
                }
            } else {
                w.cand_idx[p] = (int32_t)((uint32_t)i | kAccFlag);
                w.cand_val[p] = v;
                if constexpr (M::on) w.cand_mom[p] = up;
                const uint32_t bin = mag_key(v) >> 20;
                if (hg >= 0 && hg == g_lds) atomicAdd(&h[bin], 1u);
                else if (hg >= 0) atomicAdd(&ghist[(int64_t)hg * kRep * kBins + bin], 1u);
            }
        });
    }
    if (sampled || g_lds < 0) return;  // uniform
    __syncthreads();
    for (int b = threadIdx.x; b < kBins; b += kBlock) {
        const uint32_t c = h[b];
        if (c) atomicAdd(&ghist[(int64_t)g_lds * kRep * kBins + b], c);
    }
}

// ------------------------------------------------------------ compaction
struct ChunkView {
    int64_t g, base, end;
    int kind;
};

__device__ inline ChunkView chunk_view(const CompressWs& w, int32_t G, int64_t c)
{
    ChunkView v;
    v.g = find_bucket(w.cpre, (int64_t)G + 1, c);
    v.base = w.src_base[v.g] + (c - w.cpre[v.g]) * kChunk;
    v.end = min(v.base + kChunk, w.src_base[v.g] + w.src_len[v.g]);
    v.kind = w.src_kind[v.g];
    return v;
}

// The kPer entries of this thread in a chunk: index (with kAccFlag when r
// holds acc there) and value; bit j of the result: entry j exists.  Loads are
// clamped to the chunk's last entry and unconditional, so that all of them
// are in flight at once (a guarded load is waited for before the next).
__device__ inline uint32_t chunk_items(const CompressWs& w, const float* res, const ChunkView& v,
                                       uint32_t (&idx)[kPer], float (&val)[kPer])
{
    uint32_t valid = 0;
    if (v.kind == kSrcCand) {  // uniform
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int64_t i = min(v.base + j * kBlock + threadIdx.x, v.end - 1);
            idx[j] = (uint32_t)w.cand_idx[i];
            val[j] = w.cand_val[i];
        }
    } else {
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int64_t i = min(v.base + j * kBlock + threadIdx.x, v.end - 1);
            idx[j] = (uint32_t)i | kAccFlag;
            val[j] = res[i];
        }
    }
#pragma unroll
    for (int j = 0; j < kPer; ++j) valid |= (uint32_t)(v.base + j * kBlock + threadIdx.x < v.end) << j;
    return valid;
}

__device__ inline uint32_t group_T(const CompressWs& w, int64_t g) { return w.rank[g] > 0 ? w.prefix[g] : kNoKey; }

// Item i of chunk c lives at base + j*kBlock + tid (j < kPer): coalesced
// loads; the index order of a chunk is (j, wave, lane).
__global__ __launch_bounds__(kBlock) void k_compact_count(const float* __restrict__ res, int32_t G, CompressWs w)
{
    __shared__ uint32_t tmp[kBlock / 64 + 1];
    const int64_t nch = w.cpre[G];
    for (int64_t c = blockIdx.x; c < nch; c += gridDim.x) {
        const ChunkView v = chunk_view(w, G, c);
        const uint32_t T = group_T(w, v.g);
        uint32_t gt = 0, eq = 0;
        uint32_t id[kPer];
        float x[kPer];
        const uint32_t valid = chunk_items(w, res, v, id, x);
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const uint32_t key = mag_key(x[j]);
            const bool in = (valid >> j) & 1u;
            gt += in && key > T;
            eq += in && key == T;
        }
        uint32_t tg, te;
        block_exclusive_scan<uint32_t>(gt, tmp, &tg);
        block_exclusive_scan<uint32_t>(eq, tmp, &te);
        if (threadIdx.x == 0) {
            w.ch_gt[c] = tg;
            w.ch_eq[c] = te;
        }
    }
}

__global__ __launch_bounds__(kScanThreads) void k_chunk_scan(int32_t G, CompressWs w)
{
    const int64_t nch = w.cpre[G];
    scan_u32_to_i64(w.ch_gt, w.ch_gt_pre, nch);
    scan_u32_to_i64(w.ch_eq, w.ch_eq_pre, nch);
}

// Split chunk scan, part 1: the (gt, eq) totals of each part of kChunkPart
// chunks (coalesced reads; parts past the end give 0).
__global__ __launch_bounds__(kBlock) void k_chunk_part(int32_t G, CompressWs w)
{
    __shared__ int64_t tmp[kBlock / 64 + 1];
    const int64_t nch = w.cpre[G];
    const int64_t c0 = (int64_t)blockIdx.x * kChunkPart, c1 = min(c0 + kChunkPart, nch);
    int64_t gt = 0, eq = 0;
    for (int64_t c = c0 + threadIdx.x; c < c1; c += kBlock) {
        gt += w.ch_gt[c];
        eq += w.ch_eq[c];
    }
    int64_t tg, te;
    block_scan_excl<kBlock, int64_t>(gt, tmp, &tg);
    block_scan_excl<kBlock, int64_t>(eq, tmp, &te);
    if (threadIdx.x == 0) {
        w.cpart[2 * blockIdx.x] = tg;
        w.cpart[2 * blockIdx.x + 1] = te;
    }
}

// Split chunk scan, part 2: each workgroup adds up the parts before its own
// and scans its chunks in rounds of kBlock, coalesced; the workgroup holding
// the last chunk writes the totals.
__global__ __launch_bounds__(kBlock) void k_chunk_apply(int32_t G, CompressWs w)
{
    __shared__ int64_t tmp[kBlock / 64 + 1];
    const int64_t nch = w.cpre[G];
    const int64_t c0 = (int64_t)blockIdx.x * kChunkPart, c1 = min(c0 + kChunkPart, nch);
    int64_t bg = 0, be = 0;
    for (int64_t q = threadIdx.x; q < (int64_t)blockIdx.x; q += kBlock) {
        bg += w.cpart[2 * q];
        be += w.cpart[2 * q + 1];
    }
    int64_t rg, re;
    block_scan_excl<kBlock, int64_t>(bg, tmp, &rg);
    block_scan_excl<kBlock, int64_t>(be, tmp, &re);
    for (int64_t r0 = c0; r0 < c1; r0 += kBlock) {  // uniform
        const int64_t c = r0 + threadIdx.x;
        const int64_t g = c < c1 ? (int64_t)w.ch_gt[c] : 0, e = c < c1 ? (int64_t)w.ch_eq[c] : 0;
        int64_t tg, te;
        const int64_t xg = block_scan_excl<kBlock, int64_t>(g, tmp, &tg);
        const int64_t xe = block_scan_excl<kBlock, int64_t>(e, tmp, &te);
        if (c < c1) {
            w.ch_gt_pre[c] = rg + xg;
            w.ch_eq_pre[c] = re + xe;
        }
        rg += tg;
        re += te;
    }
    const bool last = c0 < nch ? c1 == nch : (blockIdx.x == 0 && nch == 0);
    if (last && threadIdx.x == 0) {
        w.ch_gt_pre[nch] = rg;
        w.ch_eq_pre[nch] = re;
    }
}

template <typename M>
__global__ __launch_bounds__(kBlock) void k_compact_write(float* __restrict__ res, int32_t G, CompressWs w,
                                                         int32_t* __restrict__ out_idx,
                                                         float* __restrict__ out_val, int64_t cap, M m)
{
    __shared__ uint32_t weq[kPer][kBlock / 64];
    __shared__ uint32_t wkp[kPer][kBlock / 64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
    const int64_t nch = w.cpre[G];
    for (int64_t c = blockIdx.x; c < nch; c += gridDim.x) {
        const ChunkView v = chunk_view(w, G, c);
        const uint32_t T = group_T(w, v.g);
        const uint32_t kz = w.key_z[v.g];
        const int64_t quota = w.mrem[v.g];
        const int64_t c0 = w.cpre[v.g];
        const int64_t gt_before = w.ch_gt_pre[c] - w.ch_gt_pre[c0];
        const int64_t eq_before = w.ch_eq_pre[c] - w.ch_eq_pre[c0];
        const int64_t kept_before = gt_before + (eq_before < quota ? eq_before : quota);
        uint32_t id[kPer];
        float x[kPer];
        const uint32_t valid = chunk_items(w, res, v, id, x);
        uint32_t eqb = 0, gtb = 0;
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const uint32_t key = mag_key(x[j]);
            gtb |= (uint32_t)(key > T) << j;
            eqb |= (uint32_t)(key == T) << j;
        }
        gtb &= valid;
        eqb &= valid;
        // rank of each tie among the chunk's ties, in index order
        uint32_t rk[kPer];
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const uint64_t b = __ballot((eqb >> j) & 1u);
            rk[j] = __popcll(b & below);
            if (lane == 0) weq[j][wave] = __popcll(b);
        }
        __syncthreads();
        // a tie is kept while the ties before it in the group number fewer than quota
        uint32_t keepb = gtb;
        {
            uint32_t run = 0;  // ties in the earlier slots j' < j of this chunk
#pragma unroll
            for (int j = 0; j < kPer; ++j) {
                uint32_t before = 0, tot = 0;
                for (int q = 0; q < kBlock / 64; ++q) {
                    const uint32_t cq = weq[j][q];
                    before += q < wave ? cq : 0u;
                    tot += cq;
                }
                if (((eqb >> j) & 1u) && eq_before + (int64_t)(run + before + rk[j]) < quota) keepb |= 1u << j;
                run += tot;
            }
        }
        // rank of each kept item among the chunk's kept items
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const uint64_t b = __ballot((keepb >> j) & 1u);
            rk[j] = __popcll(b & below);
            if (lane == 0) wkp[j][wave] = __popcll(b);
        }
        __syncthreads();
        {
            uint32_t run = 0;
#pragma unroll
            for (int j = 0; j < kPer; ++j) {
                uint32_t before = 0, tot = 0;
                for (int q = 0; q < kBlock / 64; ++q) {
                    const uint32_t cq = wkp[j][q];
                    before += q < wave ? cq : 0u;
                    tot += cq;
                }
                if ((valid >> j) & 1u) {
                    const uint32_t i = id[j] & ~kAccFlag;
                    const uint32_t key = mag_key(x[j]);
                    const bool zeroed = !(id[j] & kAccFlag) && key >= kz;  // pass 1 stored +0 here
                    if ((keepb >> j) & 1u) {
                        const int64_t pos = w.kpre[v.g] + kept_before + run + before + rk[j];
                        if (pos < cap) {
                            out_idx[pos] = (int32_t)i;
                            out_val[pos] = x[j];
                        }
                        if (!zeroed && !w.hold) {
                            res[i] = 0.0f;
                            if constexpr (M::on) m.u[i] = 0.0f;  // momentum masking
                        }
                    } else if (zeroed) {
                        res[i] = x[j];  // zeroed by pass 1 but not kept: give acc (and u') back
                        if constexpr (M::on) m.u[i] = w.cand_mom[v.base + j * kBlock + threadIdx.x];
                    }
                }
                run += tot;
            }
        }
        __syncthreads();  // weq / wkp are rewritten by the next chunk
    }
}

// First entry at or after position x among the ascending a[lo, hi), found
// by a whole wave: 64 evenly spaced probes per round narrow the interval
// about 64-fold (a handful of dependent loads instead of one per halving);
// every lane returns the same answer (hi when every entry is below x).
__device__ inline int64_t wave_lower_bound(const int32_t* __restrict__ a, int64_t lo, int64_t hi, int64_t x)
{
    const int lane = threadIdx.x & 63;
    while (hi - lo > 64) {  // uniform
        const int64_t step = (hi - lo + 63) / 64;
        const int64_t p = lo + lane * step;
        const bool below = p < hi && (int64_t)a[p < hi ? p : hi - 1] < x;
        const int c = __popcll(__ballot(below));  // the probes below x are a prefix of the lanes
        if (c == 0) return lo;
        const int64_t nhi = lo + (int64_t)c * step;
        lo = lo + (int64_t)(c - 1) * step + 1;
        hi = nhi < hi ? nhi : hi;
    }
    if (lo >= hi) return lo;
    const int64_t p = lo + lane;
    const bool below = p < hi && (int64_t)a[p < hi ? p : hi - 1] < x;
    return lo + __popcll(__ballot(below));
}

// Per-segment counts of the (ascending) output: one wave per segment, two
// searches for the entries below its first and past its last element.
__global__ __launch_bounds__(kBlock) void k_seg_counts(const int64_t* __restrict__ seg_off, int32_t nseg,
                                                      const int32_t* __restrict__ out_idx, CompressWs w,
                                                      int64_t* __restrict__ out_counts)
{
    const int64_t total = w.scal[0];
    const int64_t waves = (int64_t)gridDim.x * (kBlock / 64);
    const bool lead = (threadIdx.x & 63) == 0;
    for (int64_t t = (int64_t)blockIdx.x * (kBlock / 64) + (threadIdx.x >> 6); t <= nseg; t += waves) {
        if (t == nseg) {  // uniform per wave
            if (lead) out_counts[nseg] = total;
            continue;
        }
        // every index lies in [0, n): nothing below element 0, everything below n
        const int64_t x0 = seg_off[t], x1 = seg_off[t + 1];
        const int64_t a = x0 == 0 ? 0 : wave_lower_bound(out_idx, 0, total, x0);
        const int64_t b = x1 == seg_off[nseg] ? total : wave_lower_bound(out_idx, a, total, x1);
        if (lead) out_counts[t] = b - a;
    }
}

// One digit of the radix select over V virtual groups.  probe_last: the
// digit ends the probe selection (its resolve stores the probe bounds).
// skip_cand: the digit's histogram of candidate-selected groups is done.
template <int D>
static int radix_select(const float* res, int32_t V, const CompressWs& w, hipStream_t s, bool probe_last,
                        int32_t mode, bool skip_cand)
{
    k_srs_hist<D><<<kHistBlocks, kBlock, 0, s>>>(res, V, w, skip_cand ? 1 : 0);
    SGC_LAUNCH_CHECK();
    k_srs_resolve<D><<<(unsigned)V, kBlock, 0, s>>>(w, probe_last ? 1 : 0, mode);
    SGC_LAUNCH_CHECK();
    return SGC_OK;
}

size_t workspace_bytes(const sgc_layout* L, const sgc_compress_opts* o, bool mom)
{
    CompressSizes z = compress_sizes(L, o);
    Carver c(nullptr);
    CompressWs w;
    carve_compress(c, z, o->mode, mom, &w);
    return c.off;
}

// The compress step, plain (NoMom) or with momentum correction (Mom).
template <typename M>
static int run_impl(const CompressCall& a, M m)
{
    sgc_layout* L = a.L;
    const sgc_compress_opts* o = &a.o;
    const float* grad = a.grad;
    float* residual = a.residual;
    int32_t* out_idx = a.out_idx;
    float* out_val = a.out_val;
    const int64_t cap = a.cap;
    int64_t* out_counts = a.out_counts;
    uint32_t* dstatus = a.dstatus;
    const hipStream_t s = a.s;
    std::vector<int64_t> hoff = host_group_off(L, o->scope);
    const int32_t G = (int32_t)hoff.size() - 1;
    CompressSizes z = compress_sizes(L, o);
    if (!a.ws || a.ws_bytes < workspace_bytes(L, o, M::on)) return SGC_ENOSPC;
    Carver c(a.ws);
    CompressWs w;
    carve_compress(c, z, o->mode, M::on, &w);
    w.hold = a.hold ? 1u : 0u;

    DevTables* dt = nullptr;
    int rc = device_tables(L, &dt);
    if (rc) return rc;
    Groups gr = groups_of(L, dt, o->scope);
    uint32_t* status = dstatus ? dstatus : w.status;

    if (L->n == 0) {
        if (!dstatus && (rc = fill_u32(w.status, 1, 0, s))) return rc;
        if ((rc = fill_u32(w.scal, 2 * 8, 0, s))) return rc;
        k_seg_counts<<<1, kBlock, 0, s>>>(dt->seg_off, L->nseg, out_idx, w, out_counts);
        SGC_LAUNCH_CHECK();
        return SGC_OK;
    }
    const int32_t V = 2 * G;

    // 1. probe selection -> key_lo, key_z
    const int64_t hist_words = (int64_t)V * kRep * kBins;
    // exact mode, one segment per selection group: each segment keeps exactly
    // its group's k, so the output counts need no search over the indices
    const bool counts_known = o->mode == SGC_EXACT && (o->scope == SGC_PER_SEGMENT || L->nseg == 1);
    k_setup<<<(unsigned)std::min<int64_t>(cdiv(hist_words, kBlock), 256), kBlock, 0, s>>>(
        gr.off, G, o->mode, o->keep_ppm, o->sample_div, o->sample_min, w, hist_words, dstatus ? nullptr : w.status,
        counts_known ? out_counts : nullptr);
    SGC_LAUNCH_CHECK();
    if (z.S > 0) {
        unsigned pb = (unsigned)std::min<int64_t>(cdiv(z.S, kBlock), 4096);
        k_probe<M><<<pb, kBlock, 0, s>>>(grad, residual, gr.off, G, o->mode, w, z.S, m);
        SGC_LAUNCH_CHECK();
    }
    // exact mode: two digits (21 bits) place the bounds closely enough -- key_lo
    // rounded down keeps it a lower bound; sampled mode: the method's threshold
    // exactly, three digits
    if ((rc = radix_select<0>(residual, V, w, s, false, o->mode, false))) return rc;
    if ((rc = radix_select<1>(residual, V, w, s, o->mode == SGC_EXACT, o->mode, false))) return rc;
    if (o->mode != SGC_EXACT && (rc = radix_select<2>(residual, V, w, s, true, o->mode, false))) return rc;

    // 2. pass 1
    if (g_pass_start && hipEventRecord(g_pass_start, s) != hipSuccess) return SGC_EHIP;
    k_pass1<M><<<(unsigned)gr.ntiles, kPassThreads, 0, s>>>(grad, residual, gr.off, gr.tile, G, w, m);
    SGC_LAUNCH_CHECK();
    if (g_pass_stop && hipEventRecord(g_pass_stop, s) != hipSuccess) return SGC_EHIP;

    // 3. scans
    k_tile_scan1<<<(unsigned)z.NS, kBlock, 0, s>>>(gr.ntiles, w);
    SGC_LAUNCH_CHECK();
    k_tile_scan2<<<1, kScanThreads, 0, s>>>(gr.off, gr.tile, G, gr.ntiles, o->mode, z.capc, cap, w, status);
    SGC_LAUNCH_CHECK();

    // 4. gather
    k_gather<M><<<(unsigned)cdiv(gr.ntiles, kGatherTiles), kBlock, 0, s>>>(grad, residual, gr.off, gr.tile, G,
                                                                            gr.ntiles, o->mode, out_idx, out_val,
                                                                            cap, w, m);
    SGC_LAUNCH_CHECK();

    if (o->mode == SGC_EXACT) {
        // 5. exact selection over candidates (or the dense residual)
        // (the gather counted the first digit of candidate-selected groups)
        if ((rc = radix_select<0>(residual, G, w, s, false, o->mode, true))) return rc;
        if ((rc = radix_select<1>(residual, G, w, s, false, o->mode, false))) return rc;
        if ((rc = radix_select<2>(residual, G, w, s, false, o->mode, false))) return rc;
        // 6. ordered compaction
        unsigned cb = (unsigned)std::min<int64_t>(z.nch_max, 2048);
        k_compact_count<<<cb, kBlock, 0, s>>>(residual, G, w);
        SGC_LAUNCH_CHECK();
        int64_t K = 0;  // the kept total, an estimate of the candidates the scan will see
        for (int32_t g = 0; g < G; ++g) K += keep_count(hoff[g + 1] - hoff[g], o->keep_ppm);
        if (cdiv(K, kChunk) > kChunkSplit) {
            const unsigned pb = (unsigned)(cdiv(z.nch_max, kChunkPart));  // covers any chunk count
            k_chunk_part<<<pb, kBlock, 0, s>>>(G, w);
            SGC_LAUNCH_CHECK();
            k_chunk_apply<<<pb, kBlock, 0, s>>>(G, w);
            SGC_LAUNCH_CHECK();
        } else {
            k_chunk_scan<<<1, kScanThreads, 0, s>>>(G, w);
            SGC_LAUNCH_CHECK();
        }
        k_compact_write<M><<<cb, kBlock, 0, s>>>(residual, G, w, out_idx, out_val, cap, m);
        SGC_LAUNCH_CHECK();
    }
    if (counts_known) return SGC_OK;
    unsigned sb = (unsigned)std::max<int64_t>(1, std::min<int64_t>(cdiv(L->nseg + 1, kBlock / 64), 1024));
    k_seg_counts<<<sb, kBlock, 0, s>>>(dt->seg_off, L->nseg, out_idx, w, out_counts);
    SGC_LAUNCH_CHECK();
    return SGC_OK;
}

int run(const CompressCall& a)
{
    return a.mom ? run_impl(a, Mom{a.beta, a.u}) : run_impl(a, NoMom{0.0f, nullptr});
}

}  // namespace gather
}  // namespace sgc
