// compress_window.hip -- the window pipeline of sgc_compress (selection
// only between the probe's bounds; the default above about 2.5% kept and on
// vectors of 2^29 elements or more).
//
// Method ([SBC] §II Residual Accumulation and Sparse Binarization; [AH17]
// Abstract): acc = fp32(residual + grad); keep the largest-|acc| fraction
// of each selection group; send (index, value) ascending; the residual
// keeps everything else.
//
// GPU design (one HBM pass over the gradient in the common case):
//  1. probe   -- read a small sample of acc per group (runs of 16 elements)
//                and radix-select three bounds from it (top 21 key bits):
//                key_lo, a 6-sigma margin below the estimated k-th largest
//                magnitude key (the candidate bound); key_z, the estimate
//                itself (the zeroing bound); key_hi, a 6-sigma margin above
//                it (the sure bound: every key at or above it is kept).
//                Sampled mode instead takes the method's own systematic
//                sample and its exact threshold T, with key_lo = key_z = T.
//  2. pass 1  -- stream g and r once: acc = r + g; every element with
//                key >= key_lo goes into its tile's candidate region (value
//                and 16-bit offset in the tile, index order kept; staged in
//                LDS where regions are large; with the largest regions, in
//                exact mode, a 4096-bit candidate mask per tile in place of
//                the offsets); r is stored as acc, or as +0
//                for key >= key_z, so that nearly all kept entries leave the
//                residual without a second, scattered write.  Exact mode:
//                the values of the tile's window entries (key_lo <= key <
//                key_hi) also go on a short per-tile list, and the tile's
//                sure entries (key >= key_hi) are counted.  A tile whose
//                region overflows stores plain acc everywhere.
//  3. scan    -- tile counts -> offsets; per group: candidate and sure
//                totals, and how the group is selected: from its window
//                (the usual case), from all its candidates (more than k sure
//                entries), or from the whole residual (fewer than k
//                candidates: the probe misled).
//  4. select  -- the (k - sure)-th largest window key T and the quota of
//                ties at T: 2048-bin histograms over the search range
//                [key_lo, key_hi), narrowed to one bin per pass (two passes
//                for ranges up to 2^22 keys, a third only beyond); with one
//                group, the later passes read the keys the first pass
//                counted from a flat copy it made.
//  5. count   -- per tile, the entries kept without a tie (sure, key > T)
//                and the ties at T; a scan gives every tile's output offset
//                (ties are taken lowest index first).
//  6. write   -- every tile's region is read once more and the kept entries
//                written ascending (one wave per tile where regions are
//                large); the residual is zeroed only where pass 1 did not,
//                and given acc back where pass 1 zeroed an entry the exact
//                selection did not keep.
// Overflowed tiles, and every tile of a group selected from the residual,
// are worked from r (acc there) in steps 4-6, shared out over the grid.
#include "compress_path.h"

#include <cmath>

namespace sgc {
namespace window {

typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int kSuper = 1024;                     // tiles per scan super block
constexpr int kRep = 8;                          // global histogram replicas per (virtual) group
constexpr int kHistBlocks = 1024;                // workgroups of a probe histogram pass
constexpr int kTT = 64;                          // tiles per workgroup in the tile passes (one wave lane each)
constexpr int kTPer = 8;                         // items per thread per round of a tile pass, loads all in flight
constexpr int kRoundItems = kBlock * kTPer;      // items per round
constexpr int64_t kWaveWriteCap = 1024;          // regions this large take the wave-per-tile write
constexpr int64_t kStageCap = 1024;              // and pass 1 stages their candidates in LDS
constexpr int64_t kMaskCap = 2048;               // exact mode: candidate masks in place of offsets
static_assert(kMaskCap >= kStageCap && kMaskCap >= kWaveWriteCap, "masks are built staged and read by the wave write");
// Regions and window lists fill only the front of their power-of-two slots;
// a slot stride of that size would put the filled parts of every tile on the
// same HBM channels.  A pad after each slot shifts them from tile to tile.
constexpr int64_t kRegPad = 64;                  // entries after each region slot
constexpr int64_t kListPad = 32;                 // entries after each window list slot

// How a group is selected after pass 1.
constexpr int32_t kGNone = 0;    // k = 0: nothing kept
constexpr int32_t kGWindow = 1;  // the (k - sure)-th largest key of the window [key_lo, key_hi)
constexpr int32_t kGWide = 2;    // more than k sure entries: the k-th largest of all candidates
constexpr int32_t kGDense = 3;   // fewer than k candidates: the k-th largest of the whole residual

struct CompressWs {
    int64_t* k;         // [G] keep count
    int64_t* s;         // [G] probe / sample size
    int64_t* spre;      // [G+1] sample prefix
    int64_t* kpre;      // [G+1] keep-count prefix (exact output offsets)
    uint32_t* key_lo;   // [G] candidate bound (groups selected from the residual: 0)
    uint32_t* key_z;    // [G] pass-1 zeroing bound
    uint32_t* key_hi;   // [G] sure bound (kNoKey: no sure entries)
    int32_t* gmode;     // [G] kGNone / kGWindow / kGWide / kGDense
    // selection after pass 1: the k-th key is searched in [wbase, wend),
    // counted in 2048 bins of 2^wshift keys; wshift < 0: nothing left to
    // search (prefix holds T, mrem the quota of ties at T)
    uint32_t* wbase;    // [G]
    uint32_t* wend;     // [G]
    int32_t* wshift;    // [G]
    // radix-select state: 3G virtual groups in the probe (lower, zeroing and
    // sure bound), then the G groups themselves (the first G entries)
    int64_t* rank;      // [V] wanted rank (1-based); 0 = select nothing
    int64_t* cpre;      // [V+1] probe: chunk prefix over the samples
    uint32_t* prefix;   // [V] radix-select prefix -> T
    int64_t* mrem;      // [V] remaining rank -> quota of ties at T
    uint32_t* hist;     // [V * kRep * kBins] (kRep replicas spread the flush atomics)
    float* samples;     // [S]
    uint32_t* tile_cnt; // [NT] candidates (a count above tcap: the region overflowed)
    uint32_t* tile_sure;// [NT] entries at or above key_hi
    uint32_t* tile_win; // [NT] window entries (list entries past wcap are not stored)
    uint32_t* tile_sg;  // [NT] kept without a tie: sure entries and keys above T
    uint32_t* tile_eq;  // [NT] keys equal to T
    int64_t* tile_loc;  // [NT] prefix inside the super block: candidates, later tile_sg
    int64_t* tile_loc2; // [NT] prefix inside the super block: sure entries, later ties
    int64_t* sup_pre;   // [NS+1] super block prefix of the same
    int64_t* sup_pre2;  // [NS+1]
    uint16_t* reg_idx;  // [NT * tstride] offset of each candidate from its tile's first element
    uint64_t* reg_mask; // [NT * 64] large regions, exact mode, in place of reg_idx: bit i of
                        // tile t's mask marks element i of the tile a candidate
    float* reg_val;     // [NT * tstride]
    float* reg_mom;     // [NT * tstride] u' of each candidate (momentum correction only)
    float* wlist;       // [NT * wstride] window values per tile (exact mode)
    float* wflat;       // [fcap] exact mode, one group: the keys selection pass 0
                        // counted, in no order, in one segment of fcap / grid
                        // per workgroup; passes 1 and 2 (same grid) read
                        // these instead of the tiles
    uint32_t* fcnt;     // [kHistBlocks] keys in each workgroup's segment
    int64_t fcap;
    int32_t* over;      // [NT] overflowed tiles (any order)
    uint32_t* nover;    // [1] entries in over
    int32_t* dgrp;      // [G] groups selected from the residual
    int64_t* dpre;      // [G+1] their tile prefix
    int64_t* scal;      // [8]: 0 output total, 1 candidate total, 2 groups in dgrp,
                        // 4 + p: some group still searching after selection pass p,
                        // 6: a workgroup's wflat segment overflowed
    uint32_t* status;   // [1] used when the caller passes no dstatus
    uint32_t tcap;      // candidate slots per tile region (a power of two)
    uint32_t wcap;      // window list slots per tile (a power of two; exact mode)
    uint32_t tstride;   // region of tile t at t * tstride (tcap + kRegPad)
    uint32_t wstride;   // window list of tile t at t * wstride (wcap + kListPad)
    uint32_t hold;      // SGC_HOLD_KEPT: kept entries keep acc in the residual (nothing is zeroed)
};

struct CompressSizes {
    int32_t G;
    int64_t NT, NS, S, tcap, wcap, tstride, wstride;
};

// Window list slots per tile: about twice the window entries a tile
// expects -- the window [key_lo, key_hi) spans 2 x (6 sqrt(e) + 8) sampled
// keys, e = s k / m, each standing for m / s elements -- for the groups the
// probe samples (a group the probe reads whole has no sure bound; its
// tiles' lists overflow and their candidates are read from the regions).
static int64_t window_capacity(const std::vector<int64_t>& off, uint32_t ppm)
{
    double per_tile = 0.0;
    for (size_t g = 0; g + 1 < off.size(); ++g) {
        const int64_t m = off[g + 1] - off[g];
        const int64_t s = probe_count(m), k = keep_count(m, ppm);
        if (s >= m || k == 0) continue;
        const double e = (double)s * (double)k / (double)m;
        const double d = 6.0 * std::sqrt(e) + 8.0;
        per_tile = std::max(per_tile, 2.0 * d * (double)kTile / (double)s);
    }
    int64_t cap = 32;
    while (cap < 1024 && (double)cap < 2.0 * per_tile + 16.0) cap *= 2;
    return cap;
}

static CompressSizes compress_sizes(const sgc_layout* L, const sgc_compress_opts* o)
{
    CompressSizes z;
    std::vector<int64_t> off = host_group_off(L, o->scope);
    z.G = (int32_t)off.size() - 1;
    z.NT = (o->scope == SGC_GLOBAL) ? group_tiles(0, L->n) : L->seg_tile[L->nseg];
    z.NS = cdiv(z.NT, kSuper);
    z.tcap = region_capacity(o->keep_ppm);
    z.wcap = (o->mode == SGC_EXACT) ? window_capacity(off, o->keep_ppm) : 0;
    z.tstride = z.tcap + kRegPad;
    z.wstride = z.wcap ? z.wcap + kListPad : 0;
    z.S = 0;
    for (int32_t g = 0; g < z.G; ++g) {
        int64_t m = off[g + 1] - off[g];
        z.S += (o->mode == SGC_EXACT) ? probe_count(m) : sampled_count(m, o->sample_div, o->sample_min);
    }
    return z;
}

static void carve_compress(Carver& c, const CompressSizes& z, int mode, bool mom, CompressWs* w)
{
    const int64_t G = z.G, V = 3 * (int64_t)z.G;
    w->k = c.take<int64_t>(G);
    w->s = c.take<int64_t>(G);
    w->spre = c.take<int64_t>(G + 1);
    w->kpre = c.take<int64_t>(G + 1);
    w->key_lo = c.take<uint32_t>(G);
    w->key_z = c.take<uint32_t>(G);
    w->key_hi = c.take<uint32_t>(G);
    w->gmode = c.take<int32_t>(G);
    w->wbase = c.take<uint32_t>(G);
    w->wend = c.take<uint32_t>(G);
    w->wshift = c.take<int32_t>(G);
    w->rank = c.take<int64_t>(V);
    w->cpre = c.take<int64_t>(V + 1);
    w->prefix = c.take<uint32_t>(V);
    w->mrem = c.take<int64_t>(V);
    w->hist = c.take<uint32_t>(V * kRep * kBins);
    w->samples = c.take<float>(z.S);
    w->tile_cnt = c.take<uint32_t>(z.NT);
    w->tile_sure = c.take<uint32_t>(z.NT);
    w->tile_loc = c.take<int64_t>(z.NT);
    w->tile_loc2 = c.take<int64_t>(z.NT);
    w->sup_pre = c.take<int64_t>(z.NS + 1);
    w->sup_pre2 = c.take<int64_t>(z.NS + 1);
    w->tcap = (uint32_t)z.tcap;
    w->tstride = (uint32_t)z.tstride;
    // exact mode with the largest regions: a 512-byte candidate mask per
    // tile instead of 2 bytes per candidate (at 2^30 and 25% kept: 108 us
    // less per call; at 10% the expansion costs what the bytes save)
    const bool mask_mode = mode == SGC_EXACT && z.tcap >= kMaskCap;
    w->reg_idx = mask_mode ? nullptr : c.take<uint16_t>(z.NT * z.tstride);
    w->reg_mask = mask_mode ? c.take<uint64_t>(z.NT * (kTile / 64)) : nullptr;
    w->reg_val = c.take<float>(z.NT * z.tstride);
    w->reg_mom = mom ? c.take<float>(z.NT * z.tstride) : nullptr;
    w->wcap = (uint32_t)z.wcap;
    w->wstride = (uint32_t)z.wstride;
    if (mode == SGC_EXACT) {
        w->tile_win = c.take<uint32_t>(z.NT);
        w->tile_sg = c.take<uint32_t>(z.NT);
        w->tile_eq = c.take<uint32_t>(z.NT);
        w->wlist = c.take<float>(z.NT * z.wstride);
        w->fcap = G == 1 ? z.NT * z.wcap : 0;
        w->wflat = G == 1 ? c.take<float>(w->fcap) : nullptr;
        w->fcnt = G == 1 ? c.take<uint32_t>(kHistBlocks) : nullptr;
    } else {
        w->tile_win = w->tile_sg = w->tile_eq = nullptr;
        w->wlist = nullptr;
        w->wflat = nullptr;
        w->fcnt = nullptr;
        w->fcap = 0;
    }
    w->over = c.take<int32_t>(z.NT);
    w->nover = c.take<uint32_t>(1);
    w->dgrp = c.take<int32_t>(G);
    w->dpre = c.take<int64_t>(G + 1);
    w->scal = c.take<int64_t>(8);
    w->status = c.take<uint32_t>(1);
}

// Global exclusive prefix of tile t (t == NT gives the total), first and
// second prefix pair.
__device__ inline int64_t tile_prefix(const CompressWs& w, int64_t NT, int64_t t)
{
    return t >= NT ? w.sup_pre[cdiv(NT, kSuper)] : w.sup_pre[t / kSuper] + w.tile_loc[t];
}
__device__ inline int64_t tile_prefix2(const CompressWs& w, int64_t NT, int64_t t)
{
    return t >= NT ? w.sup_pre2[cdiv(NT, kSuper)] : w.sup_pre2[t / kSuper] + w.tile_loc2[t];
}

// ----------------------------------------------------------------- setup
// Every thread clears the radix-select histograms (the resolve passes leave
// them clear again); workgroup 0 clears the library's own status word (when
// the caller passes none) and the overflow-list count, and goes over the
// groups in rounds of kBlock, one thread per group: keep counts, probe
// sizes, the three ranks (lower, zeroing and sure bound) each group's probe
// selection needs, and their prefixes (workgroup scans).  counts_out (or
// NULL): exact mode with one segment per group -- the per-segment output
// counts are the groups' keep counts, written here.
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
        int64_t k = 0, sz = 0, r[3] = {0, 0, 0};  // ranks of the lower, zeroing and sure bound
        uint32_t klo = kNoKey;
        if (in) {
            const int64_t m = goff[g + 1] - goff[g];
            k = keep_count(m, ppm);
            sz = (mode == SGC_EXACT) ? probe_count(m) : sampled_count(m, div, smin);
            if (mode == SGC_EXACT) {
                if (k > 0) {
                    if (sz == m) {
                        r[0] = k;  // the probe read every element: its k-th key is the threshold
                        r[1] = w.hold ? 0 : k;
                        // no sure bound: the group is selected from all its candidates
                    } else {
                        // e: expected sampled keys above the true threshold.  The
                        // candidate bound takes a 6-sigma margin below it (a miss
                        // costs a selection from the residual), the sure bound the
                        // same margin above it (a miss costs a selection from all
                        // candidates); the zeroing bound sits at the estimate
                        // itself: either way it errs, the write pass fixes the few
                        // entries between it and the exact threshold with
                        // scattered writes
                        const double e = (double)sz * (double)k / (double)m;
                        const double d = 6.0 * sqrt(e) + 8.0;
                        const int64_t lo = (int64_t)(e + d) + 1;
                        const int64_t mid = (int64_t)(e + 0.5);
                        const double hi = e - d;
                        if (lo >= sz) klo = 0;  // the bound would be the sample minimum: take every element
                        else r[0] = lo;
                        if (mid >= 1) r[1] = mid;
                        if (w.hold) r[1] = 0;  // no zeroing bound: nothing is zeroed
                        if (hi >= 1.0) r[2] = (int64_t)hi;
                    }
                }
            } else {
                r[0] = keep_count(sz, ppm);  // the method's threshold; zeroing uses the same key
            }
        }
        int64_t c[3], csum = 0;
#pragma unroll
        for (int v = 0; v < 3; ++v) {
            c[v] = r[v] > 0 ? cdiv(sz, kChunk) : 0;
            csum += c[v];
        }
        int64_t ts, tk, tc;
        const int64_t xs = sp + block_scan_excl<kBlock, int64_t>(sz, tmp, &ts);
        const int64_t xk = kp + block_scan_excl<kBlock, int64_t>(k, tmp, &tk);
        const int64_t xc = cp + block_scan_excl<kBlock, int64_t>(csum, tmp, &tc);
        if (in) {
            w.k[g] = k;
            if (counts_out) counts_out[g] = k;
            w.s[g] = sz;
            w.spre[g] = xs;
            w.kpre[g] = xk;
            w.key_lo[g] = klo;
            w.key_z[g] = kNoKey;
            w.key_hi[g] = kNoKey;
            int64_t cc = xc;
#pragma unroll
            for (int v = 0; v < 3; ++v) {
                const int64_t vg = 3 * g + v;
                w.rank[vg] = r[v];
                w.cpre[vg] = cc;
                w.prefix[vg] = 0;
                w.mrem[vg] = r[v];
                cc += c[v];
            }
        }
        sp += ts;
        kp += tk;
        cp += tc;
    }
    if (threadIdx.x == 0) {
        w.spre[G] = sp;
        w.kpre[G] = kp;
        w.cpre[3 * G] = cp;
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
// Pick the digit holding the wanted rank (counted from the largest key) of
// (virtual) group g: sum the replicas of its histogram, scan from the top,
// clear the replicas for the next digit.  Every thread of the block calls it
// (block scan inside).  probe_last: this is the last digit of the probe
// selection; the resolving thread also stores the bound it yields (the
// chosen digits, low bits zero): virtual group 3g gives key_lo (and, in
// sampled mode, key_z = key_lo), 3g + 1 key_z and 3g + 2 key_hi.  Rounded
// down to 21 bits, key_lo stays a lower bound, and key_hi can only let a few
// more entries count as sure (the sure count is checked against k).
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
                    const int64_t grp = g / 3, v = g % 3;
                    if (v == 0) {
                        w.key_lo[grp] = key;
                        if (mode != SGC_EXACT && !w.hold) w.key_z[grp] = key;
                    } else if (v == 1) {
                        w.key_z[grp] = key;
                    } else {
                        w.key_hi[grp] = key;
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

// Probe histogram of digit D over the samples of every open virtual group,
// chunks split evenly over the workgroups; a chunk is kPer loads per
// thread, all in flight before the first is counted.
template <int D>
__global__ __launch_bounds__(kBlock) void k_srs_hist(int32_t V, CompressWs w)
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
        if (w.mrem[g] == 0) continue;
        dirty = true;
        const int64_t grp = g / 3;
        const int64_t base = w.spre[grp] + (c - w.cpre[g]) * kChunk;
        const int64_t end = w.spre[grp] + w.s[grp];
        const uint32_t pre = w.prefix[g];
        // clamped, unconditional loads: a guarded load would be waited for
        // before the next one is issued
        float x[kPer];
#pragma unroll
        for (int j = 0; j < kPer; ++j) x[j] = w.samples[min(base + j * kBlock + threadIdx.x, end - 1)];
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
// kTile): acc = r + g is formed and r is stored (acc, or +0 for key >= kz
// when the tile's candidates fit its tcap-slot region).  With momentum
// correction g is replaced by u' = beta*u + g, and u is stored like r (u',
// or +0 where r gets +0).  Returns the tile's candidate count to every
// thread and, with wl != nullptr, its window entries (klo <= key < khi):
// their count through *win and the first wcap of their values in wl, in no
// particular order (an LDS counter hands out the slots).  The tile's sure
// entries (key >= khi) are the candidates less the window entries.  Indices are 32-bit (n < 2^31); the tile base is
// uniform, so each access is a scalar base plus one 32-bit lane offset.  A
// tile that lies entirely inside its group skips every per-element range
// check.
template <int TB, int SL, typename M, typename Sink>
__device__ inline uint32_t tile_candidates(const float* __restrict__ grad, float* __restrict__ res, int32_t lo,
                                           int32_t hi, int32_t A, uint32_t klo, uint32_t kz, uint32_t khi,
                                           uint32_t tcap, M m, float* __restrict__ wl, uint32_t wcap,
                                           uint32_t* win, Sink sink)
{
    static_assert((int64_t)TB * SL * 4 == kTile, "a tile is TB threads x SL float4");
    constexpr int NW = TB / 64;
    __shared__ uint32_t wtot[SL][NW];
    __shared__ uint32_t wslot;  // next free window list slot
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (tid == 0) wslot = 0;  // used after the barrier below
    const bool full = A >= lo && (int64_t)A + kTile <= (int64_t)hi;  // uniform; 64-bit: A + kTile may reach 2^31
    const f4* rb = (const f4*)(res + A);
    const f4* gb = (const f4*)(grad + A);
    const f4* ub = M::on ? (const f4*)(m.u + A) : nullptr;  // momentum correction only
    f4 acc[SL];
    f4 um[SL];  // u' (momentum correction only)
    if (full) {
#pragma unroll
        for (int u = 0; u < SL; ++u) {
            const int o = u * TB + tid;
            const f4 rv = __builtin_nontemporal_load(rb + o);
            f4 gv = __builtin_nontemporal_load(gb + o);
            if constexpr (M::on) {
                const f4 uo = __builtin_nontemporal_load(ub + o);
#pragma unroll
                for (int j = 0; j < 4; ++j) gv[j] = mom_update(m.beta, uo[j], gv[j]);
                um[u] = gv;
            }
            acc[u] = rv + gv;
        }
    } else {
#pragma unroll
        for (int u = 0; u < SL; ++u) {
            const int32_t e = A + 4 * (u * TB + tid);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float a = 0.0f, up = 0.0f;
                if (e + j >= lo && e + j < hi) {
                    float gv = grad[e + j];
                    if constexpr (M::on) gv = mom_update(m.beta, m.u[e + j], gv);
                    up = gv;
                    a = res[e + j] + gv;
                }
                acc[u][j] = a;
                if constexpr (M::on) um[u][j] = up;
            }
        }
    }
    uint32_t flags = 0;  // 4 bits per slot
    uint32_t wflags = 0; // window entries, 4 bits per slot
    uint32_t pre[SL];
#pragma unroll
    for (int u = 0; u < SL; ++u) {
        const int32_t e = A + 4 * (u * TB + tid);
        uint32_t f = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const bool in = full || (e + j >= lo && e + j < hi);
            const uint32_t key = mag_key(acc[u][j]);
            if (in && key >= klo) f |= 1u << j;
            if (wl && in && key >= klo && key < khi) wflags |= 1u << (4 * u + j);
        }
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
    // window values to the list: a wave prefix of the lanes' counts, one LDS
    // atomic per wave for the wave's first slot (the counter was zeroed before
    // the barrier above)
    if (wl && __ballot(wflags != 0)) {  // uniform
        const uint32_t nw = __popc(wflags);
        uint32_t x = nw;  // inclusive wave scan of the lanes' counts
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const uint32_t y = __shfl_up(x, d, 64);
            if (lane >= d) x += y;
        }
        uint32_t wbase = 0;
        if (lane == 63) wbase = atomicAdd(&wslot, x);
        uint32_t slot = __shfl(wbase, 63, 64) + x - nw;
#pragma unroll
        for (int u = 0; u < SL; ++u)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if ((wflags >> (4 * u + j)) & 1u) {
                    if (slot < wcap) wl[slot] = acc[u][j];
                    ++slot;
                }
    }
    __syncthreads();  // wtot is read above and rewritten by the next call; wslot is final
    *win = wl ? wslot : 0u;
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

// Candidate masks (exact mode, large regions): a region holds the values in
// index order and bit i of the tile's 64-word mask marks element i.  Lane L of
// a wave takes word L (m): its candidates are entries pre .. pre + popc(m) - 1
// of the region, pre the candidates of the words before it (a wave scan).
__device__ inline uint32_t mask_word_prefix(uint64_t m)
{
    const int lane = threadIdx.x & 63;
    const uint32_t c = (uint32_t)__popcll(m);
    uint32_t x = c;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const uint32_t y = __shfl_up(x, d, 64);
        if (lane >= d) x += y;
    }
    return x - c;
}

__device__ inline int64_t tile_group(const int64_t* gtile, int32_t G, int64_t t)
{
    return G == 1 ? 0 : find_bucket(gtile, (int64_t)G + 1, t);
}

// First element of tile t of group g (tiles sit on a 4-aligned grid from lo & ~3).
__device__ inline int32_t tile_base(const int64_t* goff, const int64_t* gtile, int64_t g, int64_t t)
{
    return ((int32_t)goff[g] & ~3) + (int32_t)(t - gtile[g]) * (int32_t)kTile;
}

template <typename M, bool ST>
__global__ __launch_bounds__(kPassThreads) void k_pass1(const float* __restrict__ grad, float* __restrict__ res,
                                                 const int64_t* __restrict__ goff, const int64_t* __restrict__ gtile,
                                                 int32_t G, CompressWs w, M m)
{
    // ST: candidates go to LDS first and leave in one coalesced copy (large
    // regions, where direct stores would be many short scattered writes)
    __shared__ float s_val[ST ? kTile : 1];
    __shared__ uint16_t s_off[ST ? kTile : 1];
    __shared__ float s_mom[ST && M::on ? kTile : 1];
    __shared__ uint32_t s_mask[ST ? kTile / 32 : 1];  // candidate bits (mask mode)
    const bool mm = ST && w.reg_mask != nullptr;    // uniform
    if (mm && threadIdx.x < kTile / 32) s_mask[threadIdx.x] = 0;  // read after tile_candidates' barriers
    const int64_t t = blockIdx.x;
    const int64_t g = tile_group(gtile, G, t);
    const int32_t lo = (int32_t)goff[g], hi = (int32_t)goff[g + 1];
    const int32_t A = tile_base(goff, gtile, g, t);
    uint16_t* ridx = w.reg_idx ? w.reg_idx + t * w.tstride : nullptr;
    float* rval = w.reg_val + t * w.tstride;
    float* rmom = M::on ? w.reg_mom + t * w.tstride : nullptr;
    uint32_t win = 0;
    float* wl = w.wlist ? w.wlist + t * w.wstride : nullptr;  // window lists: exact mode only
    const uint32_t cnt = tile_candidates<kPassThreads, (int)(kTile / (4 * kPassThreads))>(
        grad, res, lo, hi, A, w.key_lo[g], w.key_z[g], w.key_hi[g], w.tcap, m, wl, w.wcap, &win,
        [&](uint32_t pos, int32_t i, float v, float up) {
            if (mm) atomicOr(&s_mask[(i - A) >> 5], 1u << ((i - A) & 31));
            if (pos < w.tcap) {
                if constexpr (ST) {
                    if (!mm) s_off[pos] = (uint16_t)(i - A);  // < kTile
                    s_val[pos] = v;
                    if constexpr (M::on) s_mom[pos] = up;
                } else {
                    ridx[pos] = (uint16_t)(i - A);
                    rval[pos] = v;
                    if constexpr (M::on) rmom[pos] = up;
                }
            }
        });
    if constexpr (ST) {
        // whole lines, stored nontemporally: the regions are read back only
        // after the pass, and at this volume cached stores cost the pass
        // about a tenth of its time
        __syncthreads();
        const uint32_t c = min(cnt, w.tcap);
        for (uint32_t k = threadIdx.x; k < c; k += kPassThreads) {
            if (!mm) __builtin_nontemporal_store(s_off[k], ridx + k);
            __builtin_nontemporal_store(s_val[k], rval + k);
            if constexpr (M::on) __builtin_nontemporal_store(s_mom[k], rmom + k);
        }
        if (mm && threadIdx.x < kTile / 64) {
            const uint64_t mw = (uint64_t)s_mask[2 * threadIdx.x] | ((uint64_t)s_mask[2 * threadIdx.x + 1] << 32);
            __builtin_nontemporal_store(mw, w.reg_mask + t * (kTile / 64) + threadIdx.x);
        }
    }
    if (threadIdx.x == 0) {
        w.tile_cnt[t] = cnt;
        w.tile_sure[t] = cnt - win;  // keys >= khi (sampled mode: no window, not used)
        if (wl) w.tile_win[t] = win;
    }
}

// ----------------------------------------------------------------- scans
constexpr int kScanThreads = 1024;

template <typename T>
__device__ inline T block1024_exclusive_scan(T v, T* tmp /*17*/, T* total)
{
    return block_scan_excl<kScanThreads, T>(v, tmp, total);
}

// Prefix of two per-tile counts inside each super block of kSuper tiles
// (4 per thread), and the super block sums (made prefixes by
// k_scan_supers).  list_over: append every tile whose region overflowed
// (first count above tcap) to the overflow list.
__global__ __launch_bounds__(kBlock) void k_tile_scan1(int64_t NT, const uint32_t* __restrict__ a,
                                                      const uint32_t* __restrict__ b, int64_t* __restrict__ loc_a,
                                                      int64_t* __restrict__ loc_b, int64_t* __restrict__ sup_a,
                                                      int64_t* __restrict__ sup_b, int32_t list_over, CompressWs w)
{
    __shared__ int64_t tmp[kBlock / 64 + 1];
    constexpr int per = kSuper / kBlock;
    const int64_t t0 = (int64_t)blockIdx.x * kSuper + threadIdx.x * per;
    uint32_t ca[per], cb[per];
    int64_t la = 0, lb = 0;
#pragma unroll
    for (int q = 0; q < per; ++q) {
        ca[q] = t0 + q < NT ? a[t0 + q] : 0u;
        cb[q] = t0 + q < NT ? b[t0 + q] : 0u;
        la += ca[q];
        lb += cb[q];
    }
    int64_t ta, tb;
    int64_t ra = block_exclusive_scan<int64_t>(la, tmp, &ta);
    int64_t rb = block_exclusive_scan<int64_t>(lb, tmp, &tb);
#pragma unroll
    for (int q = 0; q < per; ++q) {
        if (t0 + q < NT) {
            loc_a[t0 + q] = ra;
            loc_b[t0 + q] = rb;
        }
        ra += ca[q];
        rb += cb[q];
        if (list_over && t0 + q < NT && ca[q] > w.tcap) w.over[atomicAdd(w.nover, 1u)] = (int32_t)(t0 + q);
    }
    if (threadIdx.x == 0) {
        sup_a[blockIdx.x] = ta;
        sup_b[blockIdx.x] = tb;
    }
}

// Exclusive scan of the NS super block sums of both prefixes, in place
// (NS is at most a few hundred).
__device__ inline void scan_supers(int64_t NS, int64_t* sup_a, int64_t* sup_b, int64_t* tmp)
{
    const int64_t per = cdiv(NS, kScanThreads);
    const int64_t b = threadIdx.x * per, e = min(b + per, NS);
    int64_t la = 0, lb = 0;
    for (int64_t i = b; i < e; ++i) {
        la += sup_a[i];
        lb += sup_b[i];
    }
    int64_t ta, tb;
    int64_t ra = block1024_exclusive_scan<int64_t>(la, tmp, &ta);
    int64_t rb = block1024_exclusive_scan<int64_t>(lb, tmp, &tb);
    for (int64_t i = b; i < e; ++i) {
        const int64_t va = sup_a[i], vb = sup_b[i];
        sup_a[i] = ra;
        sup_b[i] = rb;
        ra += va;
        rb += vb;
    }
    if (threadIdx.x == 0) {
        sup_a[NS] = ta;
        sup_b[NS] = tb;
    }
    __syncthreads();  // every prefix, the totals included, is visible to the whole workgroup
}

__global__ __launch_bounds__(kScanThreads) void k_scan_supers(int64_t NT, CompressWs w)
{
    __shared__ int64_t tmp[kScanThreads / 64 + 1];
    scan_supers(cdiv(NT, kSuper), w.sup_pre, w.sup_pre2, tmp);
}

// After pass 1: the super block prefixes of the candidate and sure counts,
// then per group, one thread each, in rounds: how it is selected.
//   k = 0                      -> kGNone
//   fewer than k candidates    -> kGDense: key_lo = 0 (every element), no sure bound
//   more than k sure entries   -> kGWide: no sure bound (every candidate is in the window)
//   otherwise                  -> kGWindow: rank k - sure in the window
// The groups selected from the residual are listed with their tile prefix
// (the tile passes work their tiles from r).  Sampled mode: the output
// total (the candidates, at most cap) and the truncation flag only.
__global__ __launch_bounds__(kScanThreads) void k_tile_scan2(const int64_t* __restrict__ goff,
                                                            const int64_t* __restrict__ gtile, int32_t G, int64_t NT,
                                                            int32_t mode, int64_t cap, CompressWs w,
                                                            uint32_t* status)
{
    __shared__ int64_t tmp[kScanThreads / 64 + 1];
    scan_supers(cdiv(NT, kSuper), w.sup_pre, w.sup_pre2, tmp);
    if (mode == SGC_SAMPLED) {
        if (threadIdx.x == 0) {
            const int64_t total = tile_prefix(w, NT, NT);
            w.scal[1] = total;
            w.scal[0] = total < cap ? total : cap;
            if (total > cap) *status |= SGC_STATUS_TRUNCATED;
        }
        return;
    }
    int64_t nd = 0, dt = 0;  // groups selected from the residual, and their tiles, so far
    bool fallback = false;
    for (int64_t g0 = 0; g0 < G; g0 += kScanThreads) {
        const int64_t g = g0 + threadIdx.x;
        const bool in = g < G;
        int64_t k = 0, cg = 0, sg = 0, nt = 0;
        int32_t gm = kGNone;
        if (in) {
            k = w.k[g];
            cg = tile_prefix(w, NT, gtile[g + 1]) - tile_prefix(w, NT, gtile[g]);
            sg = tile_prefix2(w, NT, gtile[g + 1]) - tile_prefix2(w, NT, gtile[g]);
            nt = gtile[g + 1] - gtile[g];
            if (k > 0) gm = cg < k ? kGDense : sg > k ? kGWide : kGWindow;
        }
        const bool dense = gm == kGDense;
        int64_t tnd, tdt;
        const int64_t xnd = nd + block1024_exclusive_scan<int64_t>(dense ? 1 : 0, tmp, &tnd);
        const int64_t xdt = dt + block1024_exclusive_scan<int64_t>(dense ? nt : 0, tmp, &tdt);
        if (in) {
            int64_t need = 0;
            if (gm == kGWindow) {
                need = k - sg;
            } else if (gm == kGWide) {
                need = k;
                w.key_hi[g] = kNoKey;
            } else if (gm == kGDense) {
                need = k;
                w.key_lo[g] = 0;
                w.key_hi[g] = kNoKey;
                w.dgrp[xnd] = (int32_t)g;
                w.dpre[xnd] = xdt;
            }
            w.gmode[g] = gm;
            w.rank[g] = need;
            w.prefix[g] = kNoKey;
            w.mrem[g] = need;
            // the first selection pass covers [key_lo, key_hi) with 2048 bins
            const uint32_t lo = gm == kGDense ? 0u : w.key_lo[g];
            const uint32_t hi = gm == kGWindow ? w.key_hi[g] : kNoKey;
            const int L = 64 - __clzll((unsigned long long)((int64_t)hi - (int64_t)lo - 1) | 1ull);
            w.wbase[g] = lo;
            w.wend[g] = hi;
            w.wshift[g] = need > 0 ? max(L - 11, 0) : -1;
            fallback |= gm == kGDense || gm == kGWide;
        }
        nd += tnd;
        dt += tdt;
    }
    fallback = __syncthreads_or(fallback);
    if (threadIdx.x != 0) return;
    w.dpre[nd] = dt;
    w.scal[2] = nd;
    w.scal[4] = w.scal[5] = w.scal[6] = 0;
    w.scal[0] = w.kpre[G];
    if (fallback) *status |= SGC_STATUS_DENSE_PATH;
}

// ------------------------------------------------------------ tile passes
// Steps 4-7 share one shape.  Phase A: a workgroup takes kTT consecutive
// tiles; one lane per tile states how many items the tile offers (its
// region's candidates, or its window list) and a wave scan lays them end to
// end; the whole workgroup then walks them kRoundItems at a time, each
// thread loading kTPer items (clamped, unconditional loads, all in flight)
// and finding an item's tile by a binary search over the scan in LDS.
// Phase B: the tiles worked from r -- overflowed tiles, and every tile of a
// group selected from the residual -- are shared out over the whole grid,
// one tile at a time per workgroup, so that clustered inputs (runs of
// overflowed tiles) spread over every workgroup.
__device__ inline int tile_of(const uint32_t* s_pre, uint32_t e)
{
    int q = 0;  // the last tile whose items start at or before e
    for (int hb = kTT / 2; hb >= 1; hb >>= 1)
        if (e >= s_pre[q + hb]) q += hb;
    return q;
}

// Called by the 64 lanes of wave 0 (lane q = tile q): s_pre[q + 1] = items
// of tiles 0..q, s_pre[0] = 0.
__device__ inline void tile_counts_scan(uint32_t c, uint32_t* s_pre)
{
    const int q = threadIdx.x;
    uint32_t x = c;
    for (int d = 1; d < 64; d <<= 1) {
        const uint32_t y = __shfl_up(x, d, 64);
        if (q >= d) x += y;
    }
    s_pre[q + 1] = x;
    if (q == 0) s_pre[0] = 0;
}

// Wave 0: the group whose digits the workgroup's LDS histogram counts (the
// first tile's that has items; the others count straight into memory).
__device__ inline void lds_group(int32_t hg, int32_t* s_glds)
{
    const uint64_t has = __ballot(hg >= 0);
    const int first = has ? __builtin_ctzll(has) : 0;
    const int32_t gv = __shfl(hg, first, 64);
    if (threadIdx.x == 0) *s_glds = has ? gv : -1;
}

struct RTile {
    int64_t t, g;
    int64_t e0, e1;  // elements [e0, e1) of the tile inside its group
};

// The tiles of phase B: j < nover -- the overflowed tiles (those of groups
// selected from the residual are skipped here: they come with their group);
// then every tile of the nd groups selected from the residual.
__device__ inline bool rtile_at(const CompressWs& w, const int64_t* goff, const int64_t* gtile, int32_t G,
                                uint32_t nover, int64_t nd, int64_t j, RTile* r)
{
    int64_t t, g;
    if (j < (int64_t)nover) {
        t = w.over[j];
        g = tile_group(gtile, G, t);
        if (nd > 0 && w.gmode[g] == kGDense) return false;
    } else {
        const int64_t jj = j - (int64_t)nover;
        const int64_t q = find_bucket(w.dpre, nd + 1, jj);
        g = w.dgrp[q];
        t = gtile[g] + (jj - w.dpre[q]);
    }
    const int64_t A = tile_base(goff, gtile, g, t);
    r->t = t;
    r->g = g;
    r->e0 = max(A, goff[g]);
    r->e1 = min(A + kTile, goff[g + 1]);
    return true;
}

__device__ inline int64_t rtile_total(const CompressWs& w, uint32_t nover, int64_t nd)
{
    return (int64_t)nover + (nd > 0 ? w.dpre[nd] : 0);
}

// Flush the LDS histogram (nb bins) into group g's replica for this workgroup.
__device__ inline void flush_hist(const CompressWs& w, const uint32_t* h, int nb, int32_t g)
{
    if (g < 0) return;
    uint32_t* gh = w.hist + ((int64_t)g * kRep + (blockIdx.x & (kRep - 1))) * kBins;
    for (int b = threadIdx.x; b < nb; b += kBlock) {
        const uint32_t c = h[b];
        if (c) atomicAdd(&gh[b], c);
    }
}

// Selection pass 0 of a single group selected from its window: the lane's
// hits go to the workgroup's segment of the flat array (seg entries at
// dst), slots handed out by an LDS counter, one atomic per wave; entries
// past the segment are counted but not stored.
template <int N>
__device__ inline void flat_append(float* dst, uint32_t seg, uint32_t* s_cnt, const float (&v)[N],
                                   const bool (&hit)[N])
{
    const int lane = threadIdx.x & 63;
    uint32_t n = 0;
#pragma unroll
    for (int u = 0; u < N; ++u) n += hit[u] ? 1u : 0u;
    uint32_t x = n;  // inclusive wave scan of the lanes' hits
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const uint32_t y = __shfl_up(x, d, 64);
        if (lane >= d) x += y;
    }
    const uint32_t tot = __shfl(x, 63, 64);
    if (tot == 0) return;  // uniform
    uint32_t base = 0;
    if (lane == 63) base = atomicAdd(s_cnt, tot);
    uint32_t pos = __shfl(base, 63, 64) + x - n;
#pragma unroll
    for (int u = 0; u < N; ++u)
        if (hit[u]) {
            if (pos < seg) dst[pos] = v[u];
            ++pos;
        }
}

// Step 4, selection pass P (0, 1 or 2): every open group's window keys
// in its search range [wbase, wend), counted in 2048 bins -- from the window lists pass 1
// wrote (or the region, past a list's capacity, and for groups whose window
// is every candidate), and from r for the r-worked tiles.  Pass 0, phase B:
// a tile of a group selected from the residual first gets back, from its
// region, the acc (and u') that pass 1 zeroed.  Passes 1 and 2 return at
// once when no group is still searching.  A workgroup takes kTT tiles at a
// time, a grid-stride over the blocks of kTT tiles: its LDS histogram
// counts the group of its first tile (the others go straight to memory),
// flushed once at the end.  A single group selected from its window: pass 0
// also copies every key it counts into its workgroup's segment of a flat
// array, and passes 1 and 2 (launched on the same grid) each read their own
// segment (a few keys per tile) instead of walking the tiles -- unless a
// segment overflowed.
template <int P, typename M>
__global__ __launch_bounds__(kBlock) void k_tsel_hist(float* __restrict__ res, const int64_t* __restrict__ goff,
                                                     const int64_t* __restrict__ gtile, int32_t G, int64_t NT,
                                                     CompressWs w, M m)
{
    if (P > 0 && w.scal[3 + P] == 0) return;  // uniform: every group has its T
    __shared__ uint32_t s_pre[kTT + 1];
    __shared__ uint32_t s_end[kTT], s_base[kTT];
    __shared__ int32_t s_sh[kTT], s_hg[kTT], s_list[kTT];
    __shared__ uint32_t h[kBins];
    __shared__ uint32_t s_fcnt;
    for (int b = threadIdx.x; b < kBins; b += kBlock) h[b] = 0;
    if (threadIdx.x == 0) s_fcnt = 0;
    const bool flat = w.wflat != nullptr && w.gmode[0] == kGWindow;  // uniform
    const uint32_t seg = flat ? (uint32_t)(w.fcap / gridDim.x) : 0u;
    float* const fdst = flat ? w.wflat + (int64_t)blockIdx.x * seg : nullptr;
    if (P > 0 && flat && w.scal[6] == 0) {  // uniform
        const uint32_t nf = w.fcnt[blockIdx.x];
        const uint32_t base = w.wbase[0], end = w.wend[0];
        const int32_t sh = w.wshift[0];
        __syncthreads();  // h is clear
        if (sh >= 0) {
            for (uint32_t e0 = 0; e0 < nf; e0 += kRoundItems) {  // uniform
                float v[kTPer];
#pragma unroll
                for (int u = 0; u < kTPer; ++u) v[u] = fdst[min(e0 + u * kBlock + threadIdx.x, nf - 1)];
#pragma unroll
                for (int u = 0; u < kTPer; ++u) {
                    const uint32_t key = mag_key(v[u]);
                    const uint32_t bin = (key - base) >> sh;
                    const bool hit = e0 + u * kBlock + threadIdx.x < nf && key >= base && key < end &&
                                     bin < (uint32_t)kBins;
                    lds_count(h, hit, bin);
                }
            }
        }
        __syncthreads();
        flush_hist(w, h, kBins, 0);
        return;
    }
    const int32_t g_lds = (int32_t)tile_group(gtile, G, min((int64_t)blockIdx.x * kTT, NT - 1));
    uint32_t* const ghist = w.hist + (blockIdx.x & (kRep - 1)) * kBins;  // + group * kRep * kBins
    const int64_t nblk = cdiv(NT, kTT);
    for (int64_t blk = blockIdx.x; blk < nblk; blk += gridDim.x) {  // uniform
        const int64_t t0 = blk * kTT;
        __syncthreads();  // the previous block's s_* are no longer read
        if (threadIdx.x < 64) {
            const int q = threadIdx.x;
            const int64_t t = t0 + q;
            uint32_t c = 0, end = 0, base = 0;
            int32_t sh = 0, hg = -1, list = 0;
            if (t < NT) {
                const int64_t g = tile_group(gtile, G, t);
                const int32_t gm = w.gmode[g];
                const uint32_t cnt = w.tile_cnt[t];
                if ((gm == kGWindow || gm == kGWide) && cnt <= w.tcap && w.wshift[g] >= 0) {
                    const uint32_t nw = w.tile_win[t];
                    list = gm == kGWindow && nw <= w.wcap;
                    c = list ? nw : cnt;
                    end = w.wend[g];
                    base = w.wbase[g];
                    sh = w.wshift[g];
                    hg = (int32_t)g;
                }
            }
            s_end[q] = end;
            s_base[q] = base;
            s_sh[q] = sh;
            s_hg[q] = hg;
            s_list[q] = list;
            tile_counts_scan(c, s_pre);
        }
        __syncthreads();
        const uint32_t E = s_pre[kTT];
        for (uint32_t e0 = 0; e0 < E; e0 += kRoundItems) {  // uniform
            float v[kTPer];
            int qs[kTPer];
#pragma unroll
            for (int u = 0; u < kTPer; ++u) {
                const uint32_t e = min(e0 + u * kBlock + threadIdx.x, E - 1);
                const int q = tile_of(s_pre, e);
                const uint32_t jj = e - s_pre[q];
                const float* src = s_list[q] ? w.wlist + (t0 + q) * w.wstride : w.reg_val + (t0 + q) * w.tstride;
                v[u] = src[jj];
                qs[u] = e0 + u * kBlock + threadIdx.x < E ? q : -1;
            }
            bool hits[kTPer];
#pragma unroll
            for (int u = 0; u < kTPer; ++u) {
                const int q = qs[u] < 0 ? 0 : qs[u];
                const uint32_t key = mag_key(v[u]);
                const uint32_t bin = (key - s_base[q]) >> s_sh[q];  // wraps below the range: no hit
                // (bin < kBins holds for every key in range; checked all the same)
                const bool hit = qs[u] >= 0 && key >= s_base[q] && key < s_end[q] && bin < (uint32_t)kBins;
                const int32_t hg = s_hg[q];
                if (hit && hg != g_lds) atomicAdd(&ghist[(int64_t)hg * kRep * kBins + bin], 1u);
                lds_count(h, hit && hg == g_lds, bin);
                hits[u] = hit;
            }
            if (P == 0 && flat) flat_append<kTPer>(fdst, seg, &s_fcnt, v, hits);
        }
    }
    const uint32_t nover = *w.nover;
    const int64_t nd = w.scal[2];
    const int64_t nr = rtile_total(w, nover, nd);
    for (int64_t j = blockIdx.x; j < nr; j += gridDim.x) {  // uniform
        RTile rt;
        if (!rtile_at(w, goff, gtile, G, nover, nd, j, &rt)) continue;
        const int64_t g = rt.g;
        if (P == 0 && w.gmode[g] == kGDense && w.tile_cnt[rt.t] <= w.tcap) {
            // pass 1 zeroed this tile's keys >= key_z: acc (and u') back from the region
            const uint32_t kz = w.key_z[g], c = w.tile_cnt[rt.t];
            const int64_t rb = rt.t * w.tstride;
            const int32_t A = tile_base(goff, gtile, g, rt.t);
            if (w.reg_mask) {  // uniform; wave 0 walks the mask, a word per lane
                if (threadIdx.x < 64) {
                    uint64_t mw = w.reg_mask[rt.t * (kTile / 64) + threadIdx.x];
                    uint32_t q = mask_word_prefix(mw);
                    for (; mw; mw &= mw - 1, ++q) {
                        const float v = w.reg_val[rb + q];  // q < c <= tcap: the mask holds c bits
                        if (mag_key(v) >= kz) {
                            const int32_t i = A + (int32_t)threadIdx.x * 64 + __builtin_ctzll(mw);
                            res[i] = v;
                            if constexpr (M::on) m.u[i] = w.reg_mom[rb + q];
                        }
                    }
                }
            } else {
                for (uint32_t j0 = 0; j0 < c; j0 += kBlock) {  // uniform
                    const uint32_t q = j0 + threadIdx.x;
                    if (q < c) {
                        const float v = w.reg_val[rb + q];
                        if (mag_key(v) >= kz) {
                            const int32_t i = A + (int32_t)w.reg_idx[rb + q];
                            res[i] = v;
                            if constexpr (M::on) m.u[i] = w.reg_mom[rb + q];
                        }
                    }
                }
            }
            __syncthreads();  // the restored values are read below by other threads of the workgroup
        }
        const int32_t sh = w.wshift[g];
        if (sh < 0) continue;  // uniform
        const uint32_t end = w.wend[g], base = w.wbase[g];
        const bool lds = (int32_t)g == g_lds;
        for (int64_t e0 = rt.e0; e0 < rt.e1; e0 += 4 * kBlock) {  // uniform
            float x[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) x[u] = res[min(e0 + u * kBlock + (int64_t)threadIdx.x, rt.e1 - 1)];
            bool hits[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const uint32_t key = mag_key(x[u]);
                const uint32_t bin = (key - base) >> sh;
                const bool hit = e0 + u * kBlock + (int64_t)threadIdx.x < rt.e1 && key >= base && key < end &&
                                 bin < (uint32_t)kBins;
                if (hit && !lds) atomicAdd(&ghist[g * kRep * kBins + bin], 1u);
                lds_count(h, hit && lds, bin);
                hits[u] = hit;
            }
            if (P == 0 && flat) flat_append<4>(fdst, seg, &s_fcnt, x, hits);
        }
    }
    __syncthreads();
    flush_hist(w, h, kBins, g_lds);
    if (P == 0 && flat && threadIdx.x == 0) {
        w.fcnt[blockIdx.x] = s_fcnt;
        if (s_fcnt > seg) w.scal[6] = 1;  // passes 1 and 2 walk the tiles
    }
}

// The bin of selection pass P that holds the mrem-th largest key of each
// open group (one workgroup per group; clears the group's histogram): the
// search range narrows to that bin, and once the bins are single keys that
// key is T and mrem the quota of ties at T.  Records in scal[4 + P] whether
// a group is still searching.
template <int P>
__global__ __launch_bounds__(kBlock) void k_win_resolve(CompressWs w)
{
    __shared__ int64_t tmp[kBlock / 64 + 1];
    if (P > 0 && w.scal[3 + P] == 0) return;  // uniform
    const int64_t g = blockIdx.x;
    const int32_t sh = w.wshift[g];
    if (sh < 0) return;  // uniform
    constexpr int per = kBins / kBlock;
    const int64_t target = w.mrem[g];
    uint32_t* gh = w.hist + g * kRep * kBins;
    // thread t owns bins [kBins - (t+1)*per, kBins - t*per): thread 0 the largest keys
    const int top = kBins - threadIdx.x * per;
    // every load in flight first (per x kRep words, each replica's bins
    // contiguous), then the clearing stores
    uint32_t x[kRep][per];
#pragma unroll
    for (int r = 0; r < kRep; ++r)
#pragma unroll
        for (int i = 0; i < per; ++i) x[r][i] = gh[r * kBins + top - per + i];
#pragma unroll
    for (int r = 0; r < kRep; ++r)
#pragma unroll
        for (int i = 0; i < per; ++i) gh[r * kBins + top - per + i] = 0;
    uint32_t cnt[per];  // cnt[i]: bin top - 1 - i
    int64_t local = 0;
#pragma unroll
    for (int i = 0; i < per; ++i) {
        uint32_t c = 0;
#pragma unroll
        for (int r = 0; r < kRep; ++r) c += x[r][per - 1 - i];
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
                const uint32_t base = w.wbase[g] + ((uint32_t)bin << sh);
                w.mrem[g] = target - run;
                if (sh == 0) {
                    w.prefix[g] = base;
                    w.wshift[g] = -1;
                } else {
                    w.wbase[g] = base;
                    w.wend[g] = min(w.wend[g], base + (1u << sh));  // < 2^32: base < 2^31, sh <= 20
                    w.wshift[g] = max(sh - 11, 0);
                    w.scal[4 + P] = 1;
                }
                break;
            }
            run += cnt[i];
        }
    }
}

// Step 5: per tile, tile_sg = its sure entries (groups selected from the
// window) + the window keys above T, tile_eq = the window keys equal to T
// (T = kNoKey when a group needs nothing from its window).
__global__ __launch_bounds__(kBlock) void k_tile_count(const float* __restrict__ res, const int64_t* __restrict__ goff,
                                                      const int64_t* __restrict__ gtile, int32_t G, int64_t NT,
                                                      CompressWs w)
{
    __shared__ uint32_t s_pre[kTT + 1];
    __shared__ uint32_t s_khi[kTT], s_T[kTT], s_gt[kTT], s_eq[kTT], s_sure[kTT];
    __shared__ int32_t s_list[kTT], s_wr[kTT];
    __shared__ int64_t tmp[kBlock / 64 + 1];
    const int64_t t0 = (int64_t)blockIdx.x * kTT;
    if (threadIdx.x < 64) {
        const int q = threadIdx.x;
        const int64_t t = t0 + q;
        uint32_t c = 0, khi = kNoKey, T = kNoKey, sure = 0;
        int32_t list = 0, wr = 0;
        if (t < NT) {
            const int64_t g = tile_group(gtile, G, t);
            const int32_t gm = w.gmode[g];
            const uint32_t cnt = w.tile_cnt[t];
            const bool rtile = gm == kGDense || ((gm == kGWindow || gm == kGWide) && cnt > w.tcap);
            wr = !rtile;  // r-worked tiles are counted in phase B
            if ((gm == kGWindow || gm == kGWide) && !rtile) {
                sure = gm == kGWindow ? w.tile_sure[t] : 0u;
                if (w.rank[g] > 0) {
                    const uint32_t nw = w.tile_win[t];
                    list = gm == kGWindow && nw <= w.wcap;
                    c = list ? nw : cnt;
                    khi = w.key_hi[g];
                    T = w.prefix[g];
                }
            }
        }
        s_khi[q] = khi;
        s_T[q] = T;
        s_sure[q] = sure;
        s_list[q] = list;
        s_wr[q] = wr;
        s_gt[q] = 0;
        s_eq[q] = 0;
        tile_counts_scan(c, s_pre);
    }
    __syncthreads();
    const uint32_t E = s_pre[kTT];
    for (uint32_t e0 = 0; e0 < E; e0 += kRoundItems) {  // uniform
        float v[kTPer];
        int qs[kTPer];
#pragma unroll
        for (int u = 0; u < kTPer; ++u) {
            const uint32_t e = min(e0 + u * kBlock + threadIdx.x, E - 1);
            const int q = tile_of(s_pre, e);
            const uint32_t jj = e - s_pre[q];
            const float* src = s_list[q] ? w.wlist + (t0 + q) * w.wstride : w.reg_val + (t0 + q) * w.tstride;
            v[u] = src[jj];
            qs[u] = e0 + u * kBlock + threadIdx.x < E ? q : -1;
        }
#pragma unroll
        for (int u = 0; u < kTPer; ++u) {
            if (qs[u] < 0) continue;
            const int q = qs[u];
            const uint32_t key = mag_key(v[u]);
            if (key >= s_khi[q]) continue;  // a sure entry (read from a region): counted by pass 1
            if (key > s_T[q]) atomicAdd(&s_gt[q], 1u);
            else if (key == s_T[q]) atomicAdd(&s_eq[q], 1u);
        }
    }
    __syncthreads();
    if (threadIdx.x < kTT && s_wr[threadIdx.x]) {
        const int q = threadIdx.x;
        w.tile_sg[t0 + q] = s_sure[q] + s_gt[q];
        w.tile_eq[t0 + q] = s_eq[q];
    }
    const uint32_t nover = *w.nover;
    const int64_t nd = w.scal[2];
    const int64_t nr = rtile_total(w, nover, nd);
    for (int64_t j = blockIdx.x; j < nr; j += gridDim.x) {  // uniform
        RTile rt;
        if (!rtile_at(w, goff, gtile, G, nover, nd, j, &rt)) continue;
        const int64_t g = rt.g;
        const int32_t gm = w.gmode[g];
        const uint32_t klo = w.key_lo[g], khi = w.key_hi[g];
        const uint32_t T = w.rank[g] > 0 ? w.prefix[g] : kNoKey;
        int64_t gt = 0, eq = 0;
        for (int64_t e0 = rt.e0; e0 < rt.e1; e0 += 4 * kBlock) {  // uniform
            float x[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) x[u] = res[min(e0 + u * kBlock + (int64_t)threadIdx.x, rt.e1 - 1)];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const uint32_t key = mag_key(x[u]);
                const bool win = e0 + u * kBlock + (int64_t)threadIdx.x < rt.e1 && key >= klo && key < khi;
                gt += win && key > T;
                eq += win && key == T;
            }
        }
        int64_t tg, te;
        block_exclusive_scan<int64_t>(gt, tmp, &tg);
        block_exclusive_scan<int64_t>(eq, tmp, &te);
        if (threadIdx.x == 0) {
            w.tile_sg[rt.t] = (uint32_t)((gm == kGWindow ? (int64_t)w.tile_sure[rt.t] : 0) + tg);
            w.tile_eq[rt.t] = (uint32_t)te;
        }
    }
}

// Prefix of one flag per item over a round (item u of thread tid is round
// item u * kBlock + tid): the items before it in the round, and the round
// total.  One barrier; the caller separates rounds with another.
template <int P>
__device__ inline uint32_t round_prefix(const bool (&f)[P], uint32_t (&pre)[P], uint32_t (*wt)[kBlock / 64])
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
    for (int u = 0; u < P; ++u) {
        const uint64_t b = __ballot(f[u]);
        pre[u] = (uint32_t)__popcll(b & below);
        if (lane == 0) wt[u][wave] = (uint32_t)__popcll(b);
    }
    __syncthreads();
    uint32_t run = 0;
#pragma unroll
    for (int u = 0; u < P; ++u) {
        uint32_t before = 0, tot = 0;
#pragma unroll
        for (int v = 0; v < kBlock / 64; ++v) {
            const uint32_t c = wt[u][v];
            before += v < wave ? c : 0u;
            tot += c;
        }
        pre[u] += run + before;
        run += tot;
    }
    return run;
}

// Phase B of the write: the r-worked tiles (overflowed regions, groups
// selected from the residual), a workgroup per tile in rounds of kBlock
// elements, shared out over the grid.
template <typename M>
__device__ inline void write_rtiles(float* __restrict__ res, const int64_t* __restrict__ goff,
                                    const int64_t* __restrict__ gtile, int32_t G, int64_t NT, const CompressWs& w,
                                    int32_t* __restrict__ out_idx, float* __restrict__ out_val, int64_t cap, M m,
                                    uint32_t* tmp32)
{
    const uint32_t nover = *w.nover;
    const int64_t nd = w.scal[2];
    const int64_t nr = rtile_total(w, nover, nd);
    for (int64_t j = blockIdx.x; j < nr; j += gridDim.x) {  // uniform
        RTile rt;
        if (!rtile_at(w, goff, gtile, G, nover, nd, j, &rt)) continue;
        const int64_t g = rt.g, t = rt.t;
        const uint32_t klo = w.key_lo[g], khi = w.key_hi[g];
        const uint32_t T = w.rank[g] > 0 ? w.prefix[g] : kNoKey;
        const int64_t quota = w.rank[g] > 0 ? w.mrem[g] : 0;
        const int64_t sgb = tile_prefix(w, NT, t) - tile_prefix(w, NT, gtile[g]);
        const int64_t eqb = tile_prefix2(w, NT, t) - tile_prefix2(w, NT, gtile[g]);
        const int64_t base = w.kpre[g] + sgb + min(quota, eqb);
        int64_t kr = 0, qr = 0;  // kept entries and ties of the tile's earlier rounds
        for (int64_t e0 = rt.e0; e0 < rt.e1; e0 += kBlock) {  // uniform
            const int64_t e = e0 + threadIdx.x;
            const bool in = e < rt.e1;
            const int64_t ec = in ? e : rt.e1 - 1;
            const float v = res[ec];
            const uint32_t key = mag_key(v);
            const bool cand = in && key >= klo;
            const bool eq = cand && key == T && key < khi;
            uint32_t te, tk;
            const uint32_t xe = block_exclusive_scan<uint32_t>(eq ? 1u : 0u, tmp32, &te);
            const bool keep = (cand && (key >= khi || key > T)) || (eq && eqb + qr + (int64_t)xe < quota);
            const uint32_t xk = block_exclusive_scan<uint32_t>(keep ? 1u : 0u, tmp32, &tk);
            if (keep) {
                const int64_t pos = base + kr + (int64_t)xk;
                if (pos < cap) {
                    out_idx[pos] = (int32_t)e;
                    out_val[pos] = v;
                }
                if (!w.hold) {
                    res[e] = 0.0f;
                    if constexpr (M::on) m.u[e] = 0.0f;
                }
            }
            kr += tk;
            qr += te;
        }
    }
}

// Step 6: the kept entries of every tile, written ascending, and the
// residual fixes.  An entry is kept if it is sure (key >= key_hi), above T,
// or a tie at T among the first quota of its group in index order.  Phase
// A: the output position of a kept region entry is the tile's offset plus
// the kept entries before it among the workgroup's region entries (so no
// per-tile scan is needed: the per-tile counts give every tile's offset);
// likewise for the tie rank.  Phase B: r-worked tiles, a workgroup per tile
// in rounds of kBlock elements.
template <int WP, typename M>
__global__ __launch_bounds__(kBlock) void k_tile_write(float* __restrict__ res, const int64_t* __restrict__ goff,
                                                      const int64_t* __restrict__ gtile, int32_t G, int64_t NT,
                                                      CompressWs w, int32_t* __restrict__ out_idx,
                                                      float* __restrict__ out_val, int64_t cap, M m)
{
    __shared__ uint32_t s_pre[kTT + 1];
    __shared__ int64_t s_off[kTT];    // output position = s_off + kept region entries before (workgroup-wide)
    __shared__ int64_t s_toff[kTT];   // tie rank in the group = s_toff + ties before (workgroup-wide)
    __shared__ int64_t s_quota[kTT];
    __shared__ uint32_t s_T[kTT], s_khi[kTT], s_kz[kTT];
    __shared__ int32_t s_A[kTT];  // the tile's first element
    __shared__ int32_t s_anyeq;
    __shared__ uint32_t s_wk[WP][kBlock / 64], s_wq[WP][kBlock / 64];
    __shared__ uint32_t tmp32[kBlock / 64 + 1];
    const int64_t t0 = (int64_t)blockIdx.x * kTT;
    if (threadIdx.x < 64) {
        const int q = threadIdx.x;
        const int64_t t = t0 + q;
        uint32_t c = 0, T = kNoKey, khi = kNoKey, kz = kNoKey, eqc = 0;
        int64_t kept = 0, base = 0, eqb = 0, quota = 0;
        int32_t A = 0;
        if (t < NT) {
            const int64_t g = tile_group(gtile, G, t);
            const int32_t gm = w.gmode[g];
            const uint32_t cnt = w.tile_cnt[t];
            if ((gm == kGWindow || gm == kGWide) && cnt <= w.tcap) {
                c = cnt;
                A = tile_base(goff, gtile, g, t);
                T = w.rank[g] > 0 ? w.prefix[g] : kNoKey;
                quota = w.rank[g] > 0 ? w.mrem[g] : 0;
                khi = w.key_hi[g];
                kz = w.key_z[g];
                const int64_t sgb = tile_prefix(w, NT, t) - tile_prefix(w, NT, gtile[g]);
                eqb = tile_prefix2(w, NT, t) - tile_prefix2(w, NT, gtile[g]);
                eqc = w.tile_eq[t];
                kept = (int64_t)w.tile_sg[t] + min(max(quota - eqb, (int64_t)0), (int64_t)eqc);
                base = w.kpre[g] + sgb + min(quota, eqb);
            }
        }
        // workgroup-wide kept entries and ties before each tile
        int64_t xk = kept, xq = eqc;
        for (int d = 1; d < 64; d <<= 1) {
            const int64_t yk = __shfl_up(xk, d, 64), yq = __shfl_up(xq, d, 64);
            if (q >= d) {
                xk += yk;
                xq += yq;
            }
        }
        s_off[q] = base - (xk - kept);
        s_toff[q] = eqb - (xq - (int64_t)eqc);
        s_quota[q] = quota;
        s_T[q] = T;
        s_khi[q] = khi;
        s_kz[q] = kz;
        s_A[q] = A;
        const bool anyeq = __ballot(eqc > 0) != 0;
        if (q == 0) s_anyeq = anyeq;
        tile_counts_scan(c, s_pre);
    }
    __syncthreads();
    const uint32_t E = s_pre[kTT];
    const bool anyeq = s_anyeq != 0;
    int64_t K = 0, Q = 0;  // kept entries and ties of the workgroup's earlier rounds
    for (uint32_t e0 = 0; e0 < E; e0 += (kBlock * WP)) {  // uniform
        int32_t id[WP];
        float v[WP], um[WP];
        int qs[WP];
#pragma unroll
        for (int u = 0; u < WP; ++u) {
            const uint32_t e = min(e0 + u * kBlock + threadIdx.x, E - 1);
            const int q = tile_of(s_pre, e);
            const int64_t at = (t0 + q) * w.tstride + (e - s_pre[q]);
            id[u] = s_A[q] + (int32_t)w.reg_idx[at];
            v[u] = w.reg_val[at];
            um[u] = M::on ? w.reg_mom[at] : 0.0f;
            qs[u] = e0 + u * kBlock + threadIdx.x < E ? q : -1;
        }
        bool keep[WP], tie[WP];
#pragma unroll
        for (int u = 0; u < WP; ++u) {
            const int q = qs[u] < 0 ? 0 : qs[u];
            const uint32_t key = mag_key(v[u]);
            const bool ok = qs[u] >= 0;
            keep[u] = ok && (key >= s_khi[q] || key > s_T[q]);
            tie[u] = ok && key == s_T[q] && key < s_khi[q];
        }
        uint32_t pq[WP], pk[WP];
        uint32_t nq = 0;
        if (anyeq) {  // uniform
            nq = round_prefix(tie, pq, s_wq);
#pragma unroll
            for (int u = 0; u < WP; ++u) {
                const int q = qs[u] < 0 ? 0 : qs[u];
                if (tie[u] && s_toff[q] + Q + (int64_t)pq[u] < s_quota[q]) keep[u] = true;
            }
        }
        const uint32_t nk = round_prefix(keep, pk, s_wk);
#pragma unroll
        for (int u = 0; u < WP; ++u) {
            if (qs[u] < 0) continue;
            const int q = qs[u];
            const int32_t i = id[u];
            const bool zeroed = mag_key(v[u]) >= s_kz[q];  // pass 1 stored +0 here
            if (keep[u]) {
                const int64_t pos = s_off[q] + K + (int64_t)pk[u];
                if (pos < cap) {
                    out_idx[pos] = i;
                    out_val[pos] = v[u];
                }
                if (!zeroed && !w.hold) {
                    res[i] = 0.0f;
                    if constexpr (M::on) m.u[i] = 0.0f;  // momentum masking
                }
            } else if (zeroed) {
                res[i] = v[u];  // zeroed by pass 1 but not kept: acc (and u') back
                if constexpr (M::on) m.u[i] = um[u];
            }
        }
        K += nk;
        Q += nq;
        __syncthreads();  // s_wk / s_wq are rewritten by the next round
    }
    write_rtiles(res, goff, gtile, G, NT, w, out_idx, out_val, cap, m, tmp32);
}

// Step 6 where regions are large (many candidates per tile): one wave per
// tile and no workgroup barrier in phase A.  The wave walks its tile's
// region 512 entries at a time (8 per lane, all loads in flight); the
// output position of a kept entry is the tile's offset plus the kept
// entries before it in the tile (wave ballots), likewise the tie rank.
// Phase B (r-worked tiles) as in k_tile_write.
template <typename M>
__global__ __launch_bounds__(kBlock) void k_tile_write_wave(float* __restrict__ res, const int64_t* __restrict__ goff,
                                                           const int64_t* __restrict__ gtile, int32_t G, int64_t NT,
                                                           CompressWs w, int32_t* __restrict__ out_idx,
                                                           float* __restrict__ out_val, int64_t cap, M m)
{
    constexpr int U = 8;  // entries per lane per step
    __shared__ uint32_t tmp32[kBlock / 64 + 1];
    extern __shared__ uint16_t s_offs[];  // mask mode: tcap offsets per wave
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t t = (int64_t)blockIdx.x * (kBlock / 64) + wave;
    const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
    int64_t g = 0;
    int32_t gm = kGNone;
    uint32_t cnt = 0;
    if (t < NT) {  // uniform per wave
        g = tile_group(gtile, G, t);
        gm = w.gmode[g];
        cnt = w.tile_cnt[t];
    }
    const bool work = t < NT && (gm == kGWindow || gm == kGWide) && cnt <= w.tcap;  // uniform per wave
    const bool mm = w.reg_mask != nullptr;                                           // uniform
    uint16_t* const so = s_offs + (int64_t)wave * w.tcap;
    if (mm) {
        // every wave turns its tile's mask into the region's offsets in LDS
        // (a word per lane; an empty mask where the wave has no tile), then
        // the one barrier of the kernel before phase B
        uint64_t mw = work ? w.reg_mask[t * (kTile / 64) + lane] : 0ull;
        uint32_t q = mask_word_prefix(mw);
        for (; mw; mw &= mw - 1, ++q)
            if (q < w.tcap) so[q] = (uint16_t)(lane * 64 + __builtin_ctzll(mw));
        __syncthreads();
    }
    if (work) {
        {
            const uint32_t T = w.rank[g] > 0 ? w.prefix[g] : kNoKey;
            const int64_t quota = w.rank[g] > 0 ? w.mrem[g] : 0;
            const uint32_t khi = w.key_hi[g], kz = w.key_z[g];
            const int32_t A = tile_base(goff, gtile, g, t);
            const int64_t sgb = tile_prefix(w, NT, t) - tile_prefix(w, NT, gtile[g]);
            const int64_t eqb = tile_prefix2(w, NT, t) - tile_prefix2(w, NT, gtile[g]);
            int64_t pos0 = w.kpre[g] + sgb + min(quota, eqb);  // next output position of the tile
            int64_t trank = eqb;                                // tie rank of the tile's next tie
            const int64_t rb = t * w.tstride;
            for (uint32_t j0 = 0; j0 < cnt; j0 += U * 64) {  // uniform
                int32_t id[U];
                float v[U], um[U];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const uint32_t jj = min(j0 + u * 64 + lane, cnt - 1);
                    const int64_t at = rb + jj;
                    id[u] = A + (int32_t)(mm ? so[jj] : w.reg_idx[at]);
                    v[u] = w.reg_val[at];
                    um[u] = M::on ? w.reg_mom[at] : 0.0f;
                }
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const bool in = j0 + u * 64 + lane < cnt;
                    const uint32_t key = mag_key(v[u]);
                    const bool tie = in && key == T && key < khi;
                    const uint64_t tb = __ballot(tie);
                    bool keep = in && (key >= khi || key > T);
                    if (tb) {  // uniform
                        keep = keep || (tie && trank + (int64_t)__popcll(tb & below) < quota);
                        trank += __popcll(tb);
                    }
                    const uint64_t kb = __ballot(keep);
                    const int32_t i = id[u];
                    const bool zeroed = key >= kz;  // pass 1 stored +0 here
                    if (keep) {
                        const int64_t pos = pos0 + __popcll(kb & below);
                        if (pos < cap) {
                            out_idx[pos] = i;
                            out_val[pos] = v[u];
                        }
                        if (!zeroed && !w.hold) {
                            res[i] = 0.0f;
                            if constexpr (M::on) m.u[i] = 0.0f;  // momentum masking
                        }
                    } else if (in && zeroed) {
                        res[i] = v[u];  // zeroed by pass 1 but not kept: acc (and u') back
                        if constexpr (M::on) m.u[i] = um[u];
                    }
                    pos0 += __popcll(kb);
                }
            }
        }
    }
    write_rtiles(res, goff, gtile, G, NT, w, out_idx, out_val, cap, m, tmp32);
}

// Sampled mode: every candidate is kept; the output position is the tile's
// candidate prefix plus the entry's rank in its tile.  Entries past cap are
// not sent: they keep acc (and u') in the residual.
template <typename M>
__global__ __launch_bounds__(kBlock) void k_tile_write_sampled(float* __restrict__ res, const int64_t* __restrict__ goff,
                                                              const int64_t* __restrict__ gtile, int32_t G,
                                                              int64_t NT, CompressWs w, int32_t* __restrict__ out_idx,
                                                              float* __restrict__ out_val, int64_t cap, M m)
{
    __shared__ uint32_t s_pre[kTT + 1];
    __shared__ int64_t s_dst[kTT];
    __shared__ int32_t s_A[kTT];  // the tile's first element
    __shared__ uint32_t tmp32[kBlock / 64 + 1];
    const int64_t t0 = (int64_t)blockIdx.x * kTT;
    if (threadIdx.x < 64) {
        const int q = threadIdx.x;
        const int64_t t = t0 + q;
        uint32_t c = 0;
        int64_t dst = 0;
        int32_t A = 0;
        if (t < NT) {
            const uint32_t cnt = w.tile_cnt[t];
            if (cnt <= w.tcap) {
                c = cnt;
                A = tile_base(goff, gtile, tile_group(gtile, G, t), t);
            }
            dst = tile_prefix(w, NT, t);
        }
        s_dst[q] = dst;
        s_A[q] = A;
        tile_counts_scan(c, s_pre);
    }
    __syncthreads();
    const uint32_t E = s_pre[kTT];
    for (uint32_t e0 = 0; e0 < E; e0 += kRoundItems) {  // uniform
        int32_t id[kTPer];
        float v[kTPer], um[kTPer];
        int64_t ps[kTPer];
#pragma unroll
        for (int u = 0; u < kTPer; ++u) {
            const uint32_t e = min(e0 + u * kBlock + threadIdx.x, E - 1);
            const int q = tile_of(s_pre, e);
            const int64_t at = (t0 + q) * w.tstride + (e - s_pre[q]);
            id[u] = s_A[q] + (int32_t)w.reg_idx[at];
            v[u] = w.reg_val[at];
            um[u] = M::on ? w.reg_mom[at] : 0.0f;
            ps[u] = e0 + u * kBlock + threadIdx.x < E ? s_dst[q] + (e - s_pre[q]) : -1;
        }
#pragma unroll
        for (int u = 0; u < kTPer; ++u) {
            if (ps[u] < 0) continue;
            if (ps[u] < cap) {
                out_idx[ps[u]] = id[u];
                out_val[ps[u]] = v[u];
            } else {
                res[id[u]] = v[u];  // truncated: stays in the residual (and keeps its momentum)
                if constexpr (M::on) m.u[id[u]] = um[u];
            }
        }
    }
    const uint32_t nover = *w.nover;
    for (int64_t j = blockIdx.x; j < (int64_t)nover; j += gridDim.x) {  // uniform
        RTile rt;
        rtile_at(w, goff, gtile, G, nover, 0, j, &rt);
        const uint32_t klo = w.key_lo[rt.g];
        const int64_t base = tile_prefix(w, NT, rt.t);
        int64_t kr = 0;
        for (int64_t e0 = rt.e0; e0 < rt.e1; e0 += kBlock) {  // uniform
            const int64_t e = e0 + threadIdx.x;
            const bool in = e < rt.e1;
            const float v = res[in ? e : rt.e1 - 1];
            const bool cand = in && mag_key(v) >= klo;
            uint32_t tk;
            const uint32_t xk = block_exclusive_scan<uint32_t>(cand ? 1u : 0u, tmp32, &tk);
            const int64_t p = base + kr + (int64_t)xk;
            if (cand && p < cap) {
                out_idx[p] = (int32_t)e;
                out_val[p] = v;
                if (!w.hold) res[e] = 0.0f;
                if constexpr (M::on) m.u[e] = 0.0f;
            }
            kr += tk;
        }
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

// One digit of the probe's radix select over V virtual groups.
template <int D>
static int probe_digit(int32_t V, const CompressWs& w, hipStream_t s, bool probe_last, int32_t mode)
{
    k_srs_hist<D><<<kHistBlocks, kBlock, 0, s>>>(V, w);
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
    const int32_t V = 3 * G;

    // 1. probe selection -> key_lo, key_z, key_hi
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
    // exact mode: two digits (21 bits) place the bounds closely enough;
    // sampled mode: the method's threshold exactly, three digits
    if ((rc = probe_digit<0>(V, w, s, false, o->mode))) return rc;
    if ((rc = probe_digit<1>(V, w, s, o->mode == SGC_EXACT, o->mode))) return rc;
    if (o->mode != SGC_EXACT && (rc = probe_digit<2>(V, w, s, true, o->mode))) return rc;

    // 2. pass 1
    if (g_pass_start && hipEventRecord(g_pass_start, s) != hipSuccess) return SGC_EHIP;
    if (z.tcap >= kStageCap)
        k_pass1<M, true><<<(unsigned)gr.ntiles, kPassThreads, 0, s>>>(grad, residual, gr.off, gr.tile, G, w, m);
    else
        k_pass1<M, false><<<(unsigned)gr.ntiles, kPassThreads, 0, s>>>(grad, residual, gr.off, gr.tile, G, w, m);
    SGC_LAUNCH_CHECK();
    if (g_pass_stop && hipEventRecord(g_pass_stop, s) != hipSuccess) return SGC_EHIP;

    // 3. candidate and sure counts -> offsets, how each group is selected
    k_tile_scan1<<<(unsigned)z.NS, kBlock, 0, s>>>(gr.ntiles, w.tile_cnt, w.tile_sure, w.tile_loc, w.tile_loc2,
                                                     w.sup_pre, w.sup_pre2, 1, w);
    SGC_LAUNCH_CHECK();
    k_tile_scan2<<<1, kScanThreads, 0, s>>>(gr.off, gr.tile, G, gr.ntiles, o->mode, cap, w, status);
    SGC_LAUNCH_CHECK();

    const unsigned tb = (unsigned)std::max<int64_t>(1, cdiv(gr.ntiles, kTT));
    if (o->mode == SGC_EXACT) {
        // 4. selection passes over the window lists (and the r-worked tiles);
        // the third only where a search range is wider than 2^22 keys
        const unsigned hb = (unsigned)std::min<int64_t>(tb, kHistBlocks);
        k_tsel_hist<0, M><<<hb, kBlock, 0, s>>>(residual, gr.off, gr.tile, G, gr.ntiles, w, m);
        SGC_LAUNCH_CHECK();
        k_win_resolve<0><<<(unsigned)G, kBlock, 0, s>>>(w);
        SGC_LAUNCH_CHECK();
        k_tsel_hist<1, M><<<hb, kBlock, 0, s>>>(residual, gr.off, gr.tile, G, gr.ntiles, w, m);
        SGC_LAUNCH_CHECK();
        k_win_resolve<1><<<(unsigned)G, kBlock, 0, s>>>(w);
        SGC_LAUNCH_CHECK();
        k_tsel_hist<2, M><<<hb, kBlock, 0, s>>>(residual, gr.off, gr.tile, G, gr.ntiles, w, m);
        SGC_LAUNCH_CHECK();
        k_win_resolve<2><<<(unsigned)G, kBlock, 0, s>>>(w);
        SGC_LAUNCH_CHECK();
        // 5. per-tile kept counts -> offsets
        k_tile_count<<<tb, kBlock, 0, s>>>(residual, gr.off, gr.tile, G, gr.ntiles, w);
        SGC_LAUNCH_CHECK();
        k_tile_scan1<<<(unsigned)z.NS, kBlock, 0, s>>>(gr.ntiles, w.tile_sg, w.tile_eq, w.tile_loc, w.tile_loc2,
                                                         w.sup_pre, w.sup_pre2, 0, w);
        SGC_LAUNCH_CHECK();
        k_scan_supers<<<1, kScanThreads, 0, s>>>(gr.ntiles, w);
        SGC_LAUNCH_CHECK();
        // 6. write
        // items per thread per round: 4 (more workgroups resident) where
        // regions are small, 8 (fewer rounds) where they are large
        if (z.tcap >= kWaveWriteCap)
            k_tile_write_wave<M><<<(unsigned)cdiv(gr.ntiles, kBlock / 64), kBlock,
                                   w.reg_mask ? (size_t)(kBlock / 64) * z.tcap * sizeof(uint16_t) : 0, s>>>(
                residual, gr.off, gr.tile, G, gr.ntiles, w, out_idx, out_val, cap, m);
        else if (z.tcap <= 256)
            k_tile_write<4, M><<<tb, kBlock, 0, s>>>(residual, gr.off, gr.tile, G, gr.ntiles, w, out_idx, out_val,
                                                     cap, m);
        else
            k_tile_write<8, M><<<tb, kBlock, 0, s>>>(residual, gr.off, gr.tile, G, gr.ntiles, w, out_idx, out_val,
                                                     cap, m);
        SGC_LAUNCH_CHECK();
    } else {
        k_tile_write_sampled<M><<<tb, kBlock, 0, s>>>(residual, gr.off, gr.tile, G, gr.ntiles, w, out_idx, out_val,
                                                      cap, m);
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

}  // namespace window
}  // namespace sgc
