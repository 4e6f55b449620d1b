// compress.hip -- residual add + top-k selection + emission (sgc_compress).
//
// Method ([SBC] §II Residual Accumulation and Sparse Binarization; [AH17]
// Abstract): acc = fp32(residual + grad); keep the largest-|acc| fraction
// of each selection group; send (index, value) ascending; the residual
// keeps everything else.  [SBC] §II Communication Delay: between exchanges
// only residual += grad is done (SGC_ACCUMULATE_ONLY).
//
// GPU design (one HBM pass over the gradient in the common case):
//  1. probe   -- gather a small systematic sample of acc per group and
//                select from it a lower bound key_lo for the magnitude key
//                (exact mode: a margin below the estimated k-th largest;
//                sampled mode: the method's threshold itself).
//  2. pass 1  -- stream g and r once: acc = r + g, store acc to r, and emit
//                every element with key >= key_lo into a per-tile region
//                (wave ballots + LDS offsets, index order kept).
//  3. gather  -- scan the tile counts and copy the regions into one ordered
//                candidate array (a tile whose region overflowed is redone
//                from r, which now holds acc).  Sampled mode: this IS the
//                output.
//  4. select  -- exact k-th largest key per group over the candidates by a
//                3-digit radix select (11+10+10 bits, LDS histograms).  If
//                a group has fewer than k candidates (the sample misled) or
//                the candidate array is full, the group is selected and
//                compacted straight from r instead (same result, more
//                passes; reported as SGC_STATUS_DENSE_PATH).
//  5. compact -- keep key > T, plus the first `quota` entries with key == T
//                in index order (lower index wins the tie); write idx/val
//                ascending and zero the residual at the kept positions.
#include "sgc_common.h"

namespace sgc {

typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int kSrcSamples = 0, kSrcCand = 1, kSrcDense = 2;

struct CompressWs {
    int64_t* k;        // [G] keep count
    int64_t* s;        // [G] probe / sample size
    int64_t* spre;     // [G+1] sample prefix
    int64_t* kpre;     // [G+1] keep-count prefix (exact output offsets)
    uint32_t* key_lo;  // [G] pass-1 candidate bound
    int32_t* src_kind; // [G] selection source
    int64_t* src_base; // [G]
    int64_t* src_len;  // [G]
    int64_t* rank;     // [G] wanted rank (1-based); 0 = select nothing
    int64_t* cpre;     // [G+1] chunk prefix over the selection source
    uint32_t* prefix;  // [G] radix-select prefix -> T
    int64_t* mrem;     // [G] remaining rank -> quota of ties at T
    int64_t* cnt_gt;   // [G] elements with key > T
    uint32_t* hist;    // [G * kBins]
    int64_t* cstart;   // [G] candidate array start per group
    float* samples;    // [S]
    uint32_t* tile_cnt;// [NT]
    int64_t* tile_pre; // [NT+1]
    int32_t* reg_idx;  // [NT * kTileCap]
    float* reg_val;    // [NT * kTileCap]
    int32_t* cand_idx; // [capc]
    float* cand_val;   // [capc]
    uint32_t* ch_gt;   // [nch_max]
    uint32_t* ch_eq;   // [nch_max]
    int64_t* ch_gt_pre;// [nch_max+1]
    int64_t* ch_eq_pre;// [nch_max+1]
    int64_t* scal;     // [8]: 0 output total
    uint32_t* status;  // [1] used when the caller passes no dstatus
};

struct CompressSizes {
    int32_t G;
    int64_t NT, S, capc, nch_max;
};

static CompressSizes compress_sizes(const sgc_layout* L, const sgc_compress_opts* o, int64_t /*cap*/)
{
    CompressSizes z;
    std::vector<int64_t> off = host_group_off(L, o->scope);
    z.G = (int32_t)off.size() - 1;
    z.NT = (o->scope == SGC_GLOBAL) ? group_tiles(0, L->n) : L->seg_tile[L->nseg];
    z.S = 0;
    int64_t K = 0;
    for (int32_t g = 0; g < z.G; ++g) {
        int64_t m = off[g + 1] - off[g];
        z.S += (o->mode == SGC_EXACT) ? probe_count(m) : sampled_count(m, o->sample_div, o->sample_min);
        K += keep_count(m, o->keep_ppm);
    }
    z.capc = (o->mode == SGC_EXACT) ? std::min<int64_t>(L->n, 4 * K + 262144) : 0;
    z.nch_max = cdiv(L->n + z.capc + z.S, kChunk) + 2 * (int64_t)z.G + 2;
    return z;
}

static void carve_compress(Carver& c, const CompressSizes& z, int mode, CompressWs* w)
{
    const int64_t G = z.G;
    w->k = c.take<int64_t>(G);
    w->s = c.take<int64_t>(G);
    w->spre = c.take<int64_t>(G + 1);
    w->kpre = c.take<int64_t>(G + 1);
    w->key_lo = c.take<uint32_t>(G);
    w->src_kind = c.take<int32_t>(G);
    w->src_base = c.take<int64_t>(G);
    w->src_len = c.take<int64_t>(G);
    w->rank = c.take<int64_t>(G);
    w->cpre = c.take<int64_t>(G + 1);
    w->prefix = c.take<uint32_t>(G);
    w->mrem = c.take<int64_t>(G);
    w->cnt_gt = c.take<int64_t>(G);
    w->hist = c.take<uint32_t>(G * kBins);
    w->cstart = c.take<int64_t>(G);
    w->samples = c.take<float>(z.S);
    w->tile_cnt = c.take<uint32_t>(z.NT);
    w->tile_pre = c.take<int64_t>(z.NT + 1);
    w->reg_idx = c.take<int32_t>(z.NT * kTileCap);
    w->reg_val = c.take<float>(z.NT * kTileCap);
    if (mode == SGC_EXACT) {
        w->cand_idx = c.take<int32_t>(z.capc);
        w->cand_val = c.take<float>(z.capc);
        w->ch_gt = c.take<uint32_t>(z.nch_max);
        w->ch_eq = c.take<uint32_t>(z.nch_max);
        w->ch_gt_pre = c.take<int64_t>(z.nch_max + 1);
        w->ch_eq_pre = c.take<int64_t>(z.nch_max + 1);
    } else {
        w->cand_idx = nullptr;
        w->cand_val = nullptr;
        w->ch_gt = w->ch_eq = nullptr;
        w->ch_gt_pre = w->ch_eq_pre = nullptr;
    }
    w->scal = c.take<int64_t>(8);
    w->status = c.take<uint32_t>(1);
}

// ------------------------------------------------------------ accumulate
__global__ __launch_bounds__(kBlock) void k_accumulate(const float* __restrict__ g, float* __restrict__ r, int64_t n)
{
    const int64_t n4 = n >> 2;
    const f4* g4 = (const f4*)g;
    f4* r4 = (f4*)r;
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n4; i += (int64_t)gridDim.x * kBlock) {
        f4 a = __builtin_nontemporal_load(r4 + i);
        f4 b = __builtin_nontemporal_load(g4 + i);
        __builtin_nontemporal_store(a + b, r4 + i);
    }
    if (blockIdx.x == 0 && threadIdx.x < (n & 3)) {
        int64_t i = (n4 << 2) + threadIdx.x;
        r[i] = r[i] + g[i];
    }
}

// ----------------------------------------------------------------- setup
// One thread walks the groups: keep counts, sample sizes, prefixes, and
// the rank each group's probe selection needs.
__global__ void k_setup(const int64_t* __restrict__ goff, int32_t G, int32_t mode, uint32_t ppm, uint32_t div,
                        uint32_t smin, CompressWs w)
{
    if (threadIdx.x != 0 || blockIdx.x != 0) return;
    int64_t sp = 0, kp = 0, cp = 0;
    for (int32_t g = 0; g < G; ++g) {
        const int64_t m = goff[g + 1] - goff[g];
        const int64_t k = keep_count(m, ppm);
        const int64_t s = (mode == SGC_EXACT) ? probe_count(m) : sampled_count(m, div, smin);
        int64_t rank = 0;
        uint32_t klo = kNoKey;
        if (mode == SGC_EXACT) {
            if (k > 0) {
                if (s == m) {
                    rank = k;  // the probe saw every element: its k-th key is the exact threshold
                } else {
                    // expected sampled keys above the true threshold, plus a 6-sigma margin
                    double e = (double)s * (double)k / (double)m;
                    int64_t mm = (int64_t)(e + 6.0 * sqrt(e) + 8.0) + 1;
                    if (mm >= s) klo = 0;  // the bound would be the sample minimum: take every element
                    else rank = mm;
                }
            }
        } else {
            rank = keep_count(s, ppm);
        }
        w.k[g] = k;
        w.s[g] = s;
        w.spre[g] = sp;
        w.kpre[g] = kp;
        w.key_lo[g] = klo;
        w.rank[g] = rank;
        w.src_kind[g] = kSrcSamples;
        w.src_base[g] = sp;
        w.src_len[g] = rank > 0 ? s : 0;
        w.cpre[g] = cp;
        w.prefix[g] = 0;
        w.mrem[g] = rank;
        w.cnt_gt[g] = 0;
        sp += s;
        kp += k;
        cp += cdiv(w.src_len[g], kChunk);
    }
    w.spre[G] = sp;
    w.kpre[G] = kp;
    w.cpre[G] = cp;
}

// Systematic sample of acc = r + g at floor((2j+1) m / (2s)) within each group.
__global__ __launch_bounds__(kBlock) void k_probe(const float* __restrict__ grad, const float* __restrict__ res,
                                                 const int64_t* __restrict__ goff, int32_t G, CompressWs w, int64_t S)
{
    for (int64_t j = (int64_t)blockIdx.x * kBlock + threadIdx.x; j < S; j += (int64_t)gridDim.x * kBlock) {
        const int64_t g = find_bucket(w.spre, (int64_t)G + 1, j);
        const int64_t m = goff[g + 1] - goff[g];
        const int64_t s = w.s[g];
        const uint64_t jj = (uint64_t)(j - w.spre[g]);
        const int64_t pos = goff[g] + (int64_t)(((2 * jj + 1) * (uint64_t)m) / (2 * (uint64_t)s));
        w.samples[j] = res[pos] + grad[pos];
    }
}

// ----------------------------------------------------------- radix select
// Histogram of one digit over every selection source chunk whose group is
// still open and whose key matches the digits chosen so far.
template <int D>
__global__ __launch_bounds__(kBlock) void k_srs_hist(const float* __restrict__ res, int32_t G, CompressWs w)
{
    constexpr int shift = D == 0 ? 20 : D == 1 ? 10 : 0;
    constexpr uint32_t mask = D == 0 ? 0x7ffu : 0x3ffu;
    constexpr int nb = D == 0 ? 2048 : 1024;
    __shared__ uint32_t h[nb];
    const int64_t nch = w.cpre[G];
    for (int64_t c = blockIdx.x; c < nch; c += gridDim.x) {
        const int64_t g = find_bucket(w.cpre, (int64_t)G + 1, c);
        if (w.mrem[g] == 0) continue;
        for (int b = threadIdx.x; b < nb; b += kBlock) h[b] = 0;
        __syncthreads();
        const int64_t base = w.src_base[g] + (c - w.cpre[g]) * kChunk;
        const int64_t end = min(base + kChunk, w.src_base[g] + w.src_len[g]);
        const int kind = w.src_kind[g];
        const float* src = kind == kSrcSamples ? w.samples : kind == kSrcCand ? w.cand_val : res;
        const uint32_t pre = w.prefix[g];
        for (int64_t i = base + threadIdx.x; i < end; i += kBlock) {
            const uint32_t key = mag_key(src[i]);
            if (D == 0 || (key >> (shift + 10)) == pre) atomicAdd(&h[(key >> shift) & mask], 1u);
        }
        __syncthreads();
        uint32_t* gh = w.hist + (int64_t)g * kBins;
        for (int b = threadIdx.x; b < nb; b += kBlock)
            if (h[b]) atomicAdd(&gh[b], h[b]);
        __syncthreads();
    }
}

// Pick the digit holding the wanted rank (counted from the largest key).
template <int D>
__global__ __launch_bounds__(kBlock) void k_srs_resolve(int32_t G, CompressWs w)
{
    constexpr int nb = D == 0 ? 2048 : 1024;
    constexpr int bits = D == 0 ? 11 : 10;
    constexpr int per = nb / kBlock;
    __shared__ int64_t tmp[kBlock / 64 + 1];
    const int64_t g = blockIdx.x;
    const int64_t target = w.mrem[g];
    if (target == 0) return;  // uniform per block
    uint32_t* gh = w.hist + g * kBins;
    // thread t owns bins [nb - (t+1)*per, nb - t*per): thread 0 the largest keys
    const int top = nb - threadIdx.x * per;
    int64_t local = 0;
#pragma unroll
    for (int i = 1; i <= per; ++i) local += gh[top - i];
    int64_t total;
    const int64_t above = block_exclusive_scan<int64_t>(local, tmp, &total);
    if (above < target && above + local >= target) {
        int64_t run = above;
        for (int i = 1; i <= per; ++i) {
            const int bin = top - i;
            const int64_t c = gh[bin];
            if (run + c >= target) {
                w.prefix[g] = (w.prefix[g] << bits) | (uint32_t)bin;
                w.cnt_gt[g] += run;
                w.mrem[g] = target - run;
                break;
            }
            run += c;
        }
    }
#pragma unroll
    for (int i = 1; i <= per; ++i) gh[top - i] = 0;
}

// After the probe selection: pass-1 bound of every group that selected.
__global__ void k_probe_done(int32_t G, CompressWs w)
{
    for (int32_t g = blockIdx.x * kBlock + threadIdx.x; g < G; g += gridDim.x * kBlock)
        if (w.rank[g] > 0) w.key_lo[g] = w.prefix[g];
}

// ---------------------------------------------------------------- pass 1
// Writes the candidates of one tile in index order through `sink(pos, i, v)`.
// ADD: acc = r + g is formed and stored to r (pass 1); otherwise r already
// holds acc (redo of an overflowed tile).  Returns the tile's candidate count
// to every thread.
template <bool ADD, typename Sink>
__device__ inline uint32_t tile_candidates(const float* __restrict__ grad, float* __restrict__ res, int64_t lo,
                                           int64_t hi, int64_t A, uint32_t klo, Sink sink)
{
    __shared__ uint32_t wtot[kSlots][kBlock / 64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    f4 acc[kSlots];
#pragma unroll
    for (int u = 0; u < kSlots; ++u) {
        const int64_t e = A + 4 * ((int64_t)u * kBlock + tid);
        if (e >= lo && e + 4 <= hi) {
            if (ADD) {
                f4 rv = __builtin_nontemporal_load((const f4*)(res + e));
                f4 gv = __builtin_nontemporal_load((const f4*)(grad + e));
                acc[u] = rv + gv;
            } else {
                acc[u] = *(const f4*)(res + e);
            }
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float a = 0.0f;
                if (e + j >= lo && e + j < hi) a = ADD ? res[e + j] + grad[e + j] : res[e + j];
                acc[u][j] = a;
            }
        }
    }
    if (ADD) {
#pragma unroll
        for (int u = 0; u < kSlots; ++u) {
            const int64_t e = A + 4 * ((int64_t)u * kBlock + tid);
            if (e >= lo && e + 4 <= hi) {
                __builtin_nontemporal_store(acc[u], (f4*)(res + e));
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (e + j >= lo && e + j < hi) res[e + j] = acc[u][j];
            }
        }
    }
    uint32_t flags[kSlots], pre[kSlots];
#pragma unroll
    for (int u = 0; u < kSlots; ++u) {
        const int64_t e = A + 4 * ((int64_t)u * kBlock + tid);
        uint32_t f = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (e + j >= lo && e + j < hi && mag_key(acc[u][j]) >= klo) f |= 1u << j;
        flags[u] = f;
        const uint32_t cnt = __popc(f);
        const uint64_t b0 = __ballot(cnt & 1u), b1 = __ballot(cnt & 2u), b2 = __ballot(cnt & 4u);
        const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
        pre[u] = __popcll(b0 & below) + 2u * __popcll(b1 & below) + 4u * __popcll(b2 & below);
        if (lane == 0) wtot[u][wave] = __popcll(b0) + 2u * __popcll(b1) + 4u * __popcll(b2);
    }
    __syncthreads();
    uint32_t run = 0, base[kSlots];
#pragma unroll
    for (int u = 0; u < kSlots; ++u) {
        for (int v = 0; v < kBlock / 64; ++v) {
            if (v == wave) base[u] = run;
            run += wtot[u][v];
        }
    }
    __syncthreads();  // wtot is reused by the next call in this block
#pragma unroll
    for (int u = 0; u < kSlots; ++u) {
        if (!flags[u]) continue;
        const int64_t e = A + 4 * ((int64_t)u * kBlock + tid);
        uint32_t pos = base[u] + pre[u];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (flags[u] & (1u << j)) sink(pos++, e + j, acc[u][j]);
    }
    return run;
}

__device__ inline int64_t tile_group(const int64_t* gtile, int32_t G, int64_t t)
{
    return G == 1 ? 0 : find_bucket(gtile, (int64_t)G + 1, t);
}

__global__ __launch_bounds__(kBlock) void k_pass1(const float* __restrict__ grad, float* __restrict__ res,
                                                 const int64_t* __restrict__ goff, const int64_t* __restrict__ gtile,
                                                 int32_t G, CompressWs w)
{
    const int64_t t = blockIdx.x;
    const int64_t g = tile_group(gtile, G, t);
    const int64_t lo = goff[g], hi = goff[g + 1];
    const int64_t A = (lo & ~(int64_t)3) + (t - gtile[g]) * kTile;
    int32_t* ridx = w.reg_idx + t * kTileCap;
    float* rval = w.reg_val + t * kTileCap;
    const uint32_t cnt = tile_candidates<true>(grad, res, lo, hi, A, w.key_lo[g],
                                               [&](uint32_t pos, int64_t i, float v) {
                                                   if (pos < (uint32_t)kTileCap) {
                                                       ridx[pos] = (int32_t)i;
                                                       rval[pos] = v;
                                                   }
                                               });
    if (threadIdx.x == 0) w.tile_cnt[t] = cnt;
}

// --------------------------------------------------------- scans (1 block)
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

// Tile-count prefix, then per group: candidate count, source of the main
// selection (candidates, or the dense residual), and chunk prefix.
__global__ __launch_bounds__(kScanThreads) void k_tile_scan(const int64_t* __restrict__ goff,
                                                           const int64_t* __restrict__ gtile, int32_t G, int64_t NT,
                                                           int32_t mode, int64_t capc, int64_t cap, CompressWs w,
                                                           uint32_t* status)
{
    scan_u32_to_i64(w.tile_cnt, w.tile_pre, NT);
    if (threadIdx.x != 0) return;
    if (mode == SGC_SAMPLED) {
        const int64_t total = w.tile_pre[NT];
        w.scal[0] = total < cap ? total : cap;
        if (total > cap) *status |= SGC_STATUS_TRUNCATED;
        return;
    }
    int64_t used = 0, cp = 0;
    bool dense = false;
    for (int32_t g = 0; g < G; ++g) {
        const int64_t cg = w.tile_pre[gtile[g + 1]] - w.tile_pre[gtile[g]];
        const int64_t k = w.k[g];
        int kind;
        int64_t base, len;
        if (k == 0) {
            kind = kSrcCand;
            base = used;
            len = 0;
        } else if (cg >= k && used + cg <= capc) {
            kind = kSrcCand;
            base = used;
            len = cg;
            used += cg;
        } else {
            kind = kSrcDense;
            base = goff[g];
            len = goff[g + 1] - goff[g];
            dense = true;
        }
        w.cstart[g] = base;
        w.src_kind[g] = kind;
        w.src_base[g] = base;
        w.src_len[g] = len;
        w.rank[g] = k;
        w.prefix[g] = 0;
        w.mrem[g] = k;
        w.cnt_gt[g] = 0;
        w.cpre[g] = cp;
        cp += cdiv(len, kChunk);
    }
    w.cpre[G] = cp;
    w.scal[0] = w.kpre[G];
    if (dense) *status |= SGC_STATUS_DENSE_PATH;
}

// Region copy (or redo of an overflowed tile) into the ordered candidate
// array (exact) or straight into the output (sampled, truncated at cap).
__global__ __launch_bounds__(kBlock) void k_gather(const float* __restrict__ grad, float* __restrict__ res,
                                                  const int64_t* __restrict__ goff, const int64_t* __restrict__ gtile,
                                                  int32_t G, int32_t mode, int32_t* __restrict__ out_idx,
                                                  float* __restrict__ out_val, int64_t cap, CompressWs w)
{
    const int64_t t = blockIdx.x;
    const uint32_t c = w.tile_cnt[t];
    if (c == 0) return;
    const int64_t g = tile_group(gtile, G, t);
    int64_t dst;
    int32_t* di;
    float* dv;
    int64_t lim;
    const bool sampled = mode == SGC_SAMPLED;
    if (sampled) {
        dst = w.tile_pre[t];
        di = out_idx;
        dv = out_val;
        lim = cap;
    } else {
        if (w.src_kind[g] != kSrcCand) return;
        dst = w.cstart[g] + w.tile_pre[t] - w.tile_pre[gtile[g]];
        di = w.cand_idx;
        dv = w.cand_val;
        lim = INT64_MAX;
    }
    if (dst >= lim) return;
    if (c <= (uint32_t)kTileCap) {
        const int32_t* ri = w.reg_idx + t * kTileCap;
        const float* rv = w.reg_val + t * kTileCap;
        for (uint32_t j = threadIdx.x; j < c; j += kBlock) {
            const int64_t p = dst + j;
            if (p >= lim) break;
            const int32_t i = ri[j];
            di[p] = i;
            dv[p] = rv[j];
            if (sampled) res[i] = 0.0f;
        }
    } else {
        const int64_t lo = goff[g], hi = goff[g + 1];
        const int64_t A = (lo & ~(int64_t)3) + (t - gtile[g]) * kTile;
        tile_candidates<false>(grad, res, lo, hi, A, w.key_lo[g], [&](uint32_t pos, int64_t i, float v) {
            const int64_t p = dst + pos;
            if (p < lim) {
                di[p] = (int32_t)i;
                dv[p] = v;
                if (sampled) res[i] = 0.0f;
            }
        });
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

__device__ inline void chunk_item(const CompressWs& w, const float* res, const int64_t* goff, const ChunkView& v,
                                  int64_t i, int32_t* idx, float* val)
{
    if (v.kind == kSrcCand) {
        *idx = w.cand_idx[i];
        *val = w.cand_val[i];
    } else {
        *idx = (int32_t)i;
        *val = res[i];
    }
}

__device__ inline uint32_t group_T(const CompressWs& w, int64_t g) { return w.rank[g] > 0 ? w.prefix[g] : kNoKey; }

__global__ __launch_bounds__(kBlock) void k_compact_count(const float* __restrict__ res, const int64_t* goff,
                                                         int32_t G, CompressWs w)
{
    __shared__ uint32_t tmp[kBlock / 64 + 1];
    const int64_t nch = w.cpre[G];
    for (int64_t c = blockIdx.x; c < nch; c += gridDim.x) {
        const ChunkView v = chunk_view(w, G, c);
        const uint32_t T = group_T(w, v.g);
        uint32_t gt = 0, eq = 0;
        const int64_t b = v.base + (int64_t)threadIdx.x * kPer;
        for (int j = 0; j < kPer; ++j) {
            const int64_t i = b + j;
            if (i < v.end) {
                int32_t id;
                float x;
                chunk_item(w, res, goff, v, i, &id, &x);
                const uint32_t key = mag_key(x);
                gt += key > T;
                eq += key == T;
            }
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

__global__ __launch_bounds__(kBlock) void k_compact_write(float* __restrict__ res, const int64_t* goff, int32_t G,
                                                         CompressWs w, int32_t* __restrict__ out_idx,
                                                         float* __restrict__ out_val, int64_t cap)
{
    __shared__ uint32_t tmp[kBlock / 64 + 1];
    const int64_t nch = w.cpre[G];
    for (int64_t c = blockIdx.x; c < nch; c += gridDim.x) {
        const ChunkView v = chunk_view(w, G, c);
        const uint32_t T = group_T(w, v.g);
        const int64_t quota = w.mrem[v.g];
        const int64_t c0 = w.cpre[v.g];
        const int64_t gt_before = w.ch_gt_pre[c] - w.ch_gt_pre[c0];
        const int64_t eq_before = w.ch_eq_pre[c] - w.ch_eq_pre[c0];
        const int64_t kept_before = gt_before + (eq_before < quota ? eq_before : quota);
        int32_t id[kPer];
        float x[kPer];
        uint32_t key[kPer];
        uint32_t eq = 0;
        const int64_t b = v.base + (int64_t)threadIdx.x * kPer;
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int64_t i = b + j;
            key[j] = kNoKey;
            if (i < v.end) {
                chunk_item(w, res, goff, v, i, &id[j], &x[j]);
                key[j] = mag_key(x[j]);
                eq += key[j] == T;
            }
        }
        uint32_t tot;
        uint32_t eq_rank = block_exclusive_scan<uint32_t>(eq, tmp, &tot);
        uint32_t keep = 0, nkeep = 0;
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            bool k = false;
            if (key[j] != kNoKey) {
                if (key[j] > T) k = true;
                else if (key[j] == T) {
                    k = eq_before + (int64_t)eq_rank < quota;
                    ++eq_rank;
                }
            }
            keep |= (uint32_t)k << j;
            nkeep += k;
        }
        uint32_t kept_rank = block_exclusive_scan<uint32_t>(nkeep, tmp, &tot);
        int64_t pos = w.kpre[v.g] + kept_before + kept_rank;
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            if ((keep & (1u << j)) && pos < cap) {
                out_idx[pos] = id[j];
                out_val[pos] = x[j];
                res[id[j]] = 0.0f;
                ++pos;
            }
        }
    }
}

// Per-segment counts of the (ascending) output by binary search.
__global__ void k_seg_counts(const int64_t* __restrict__ seg_off, int32_t nseg, const int32_t* __restrict__ out_idx,
                             CompressWs w, int64_t* __restrict__ out_counts)
{
    const int64_t total = w.scal[0];
    for (int64_t t = (int64_t)blockIdx.x * kBlock + threadIdx.x; t <= nseg; t += (int64_t)gridDim.x * kBlock) {
        if (t == nseg) {
            out_counts[nseg] = total;
            continue;
        }
        // first entry >= seg_off[t] and first entry >= seg_off[t+1]
        int64_t a0 = 0, a1 = total;
        const int64_t x0 = seg_off[t];
        while (a0 < a1) {
            int64_t m = (a0 + a1) >> 1;
            if (out_idx[m] < x0) a0 = m + 1; else a1 = m;
        }
        int64_t b0 = a0, b1 = total;
        const int64_t x1 = seg_off[t + 1];
        while (b0 < b1) {
            int64_t m = (b0 + b1) >> 1;
            if (out_idx[m] < x1) b0 = m + 1; else b1 = m;
        }
        out_counts[t] = b0 - a0;
    }
}

template <int D>
static int radix_select(const float* res, int32_t G, int64_t nch_max, const CompressWs& w, hipStream_t s)
{
    unsigned blocks = (unsigned)std::min<int64_t>(std::max<int64_t>(nch_max, 1), 2048);
    k_srs_hist<D><<<blocks, kBlock, 0, s>>>(res, G, w);
    SGC_LAUNCH_CHECK();
    k_srs_resolve<D><<<(unsigned)G, kBlock, 0, s>>>(G, w);
    SGC_LAUNCH_CHECK();
    return SGC_OK;
}

static int select_all(const float* res, int32_t G, int64_t nch_max, const CompressWs& w, hipStream_t s)
{
    int rc;
    if ((rc = radix_select<0>(res, G, nch_max, w, s))) return rc;
    if ((rc = radix_select<1>(res, G, nch_max, w, s))) return rc;
    return radix_select<2>(res, G, nch_max, w, s);
}

}  // namespace sgc

using namespace sgc;

static bool opts_ok(const sgc_layout* L, const sgc_compress_opts* o)
{
    if (!L || !o) return false;
    if (o->mode != SGC_EXACT && o->mode != SGC_SAMPLED && o->mode != SGC_ACCUMULATE_ONLY) return false;
    if (o->scope != SGC_GLOBAL && o->scope != SGC_PER_SEGMENT) return false;
    if (o->keep_ppm > 1000000) return false;
    if (o->mode == SGC_SAMPLED && o->sample_div == 0) return false;
    return true;
}

extern "C" size_t sgc_compress_workspace(const sgc_layout* L, const sgc_compress_opts* o, int64_t cap)
{
    if (!opts_ok(L, o) || cap < 0) return 0;
    if (o->mode == SGC_ACCUMULATE_ONLY) return 0;
    CompressSizes z = compress_sizes(L, o, cap);
    Carver c(nullptr);
    CompressWs w;
    carve_compress(c, z, o->mode, &w);
    return c.off;
}

extern "C" int sgc_compress(const sgc_layout* Lc, const sgc_compress_opts* o, const float* grad, float* residual,
                            int32_t* out_idx, float* out_val, int64_t cap, int64_t* out_counts, uint32_t* dstatus,
                            void* ws, size_t ws_bytes, sgc_stream_t stream)
{
    sgc_layout* L = const_cast<sgc_layout*>(Lc);
    if (!opts_ok(L, o)) return SGC_EINVAL;
    if ((L->n > 0 && (!grad || !residual)) || !aligned16(grad) || !aligned16(residual)) return SGC_EINVAL;
    hipStream_t s = (hipStream_t)stream;
    if (o->mode == SGC_ACCUMULATE_ONLY) {
        if (L->n == 0) return SGC_OK;
        int64_t blocks = std::min<int64_t>(cdiv(std::max<int64_t>(L->n >> 2, 1), kBlock), 8192);
        k_accumulate<<<(unsigned)blocks, kBlock, 0, s>>>(grad, residual, L->n);
        SGC_LAUNCH_CHECK();
        return SGC_OK;
    }
    if (!out_counts || cap < 0 || cap >= ((int64_t)1 << 31)) return SGC_EINVAL;
    if (cap > 0 && (!out_idx || !out_val)) return SGC_EINVAL;
    std::vector<int64_t> hoff = host_group_off(L, o->scope);
    const int32_t G = (int32_t)hoff.size() - 1;
    if (o->mode == SGC_EXACT) {
        int64_t K = 0;
        for (int32_t g = 0; g < G; ++g) K += keep_count(hoff[g + 1] - hoff[g], o->keep_ppm);
        if (cap < K) return SGC_EINVAL;
    }
    CompressSizes z = compress_sizes(L, o, cap);
    {
        Carver c(nullptr);
        CompressWs w0;
        carve_compress(c, z, o->mode, &w0);
        if (!ws || ws_bytes < c.off) return SGC_ENOSPC;
    }
    Carver c(ws);
    CompressWs w;
    carve_compress(c, z, o->mode, &w);

    DevTables* dt = nullptr;
    int rc = device_tables(L, &dt);
    if (rc) return rc;
    Groups gr = groups_of(L, dt, o->scope);
    uint32_t* status = dstatus ? dstatus : w.status;
    if (!dstatus && (rc = fill_u32(w.status, 1, 0, s))) return rc;

    if (L->n == 0) {
        if ((rc = fill_u32(w.scal, 2, 0, s))) return rc;
        k_seg_counts<<<1, kBlock, 0, s>>>(dt->seg_off, L->nseg, out_idx, w, out_counts);
        SGC_LAUNCH_CHECK();
        return SGC_OK;
    }

    // 1. probe selection -> key_lo
    k_setup<<<1, 64, 0, s>>>(gr.off, G, o->mode, o->keep_ppm, o->sample_div, o->sample_min, w);
    SGC_LAUNCH_CHECK();
    if ((rc = fill_u32(w.hist, (int64_t)G * kBins, 0, s))) return rc;
    if (z.S > 0) {
        unsigned pb = (unsigned)std::min<int64_t>(cdiv(z.S, kBlock), 4096);
        k_probe<<<pb, kBlock, 0, s>>>(grad, residual, gr.off, G, w, z.S);
        SGC_LAUNCH_CHECK();
    }
    if ((rc = select_all(residual, G, cdiv(z.S, kChunk) + G + 1, w, s))) return rc;
    k_probe_done<<<(unsigned)std::max<int64_t>(1, std::min<int64_t>(cdiv(G, kBlock), 1024)), kBlock, 0, s>>>(G, w);
    SGC_LAUNCH_CHECK();

    // 2. pass 1
    k_pass1<<<(unsigned)gr.ntiles, kBlock, 0, s>>>(grad, residual, gr.off, gr.tile, G, w);
    SGC_LAUNCH_CHECK();

    // 3. gather
    k_tile_scan<<<1, kScanThreads, 0, s>>>(gr.off, gr.tile, G, gr.ntiles, o->mode, z.capc, cap, w, status);
    SGC_LAUNCH_CHECK();
    k_gather<<<(unsigned)gr.ntiles, kBlock, 0, s>>>(grad, residual, gr.off, gr.tile, G, o->mode, out_idx, out_val,
                                                    cap, w);
    SGC_LAUNCH_CHECK();

    if (o->mode == SGC_EXACT) {
        // 4. exact selection over candidates (or the dense residual)
        if ((rc = select_all(residual, G, z.nch_max, w, s))) return rc;
        // 5. ordered compaction
        unsigned cb = (unsigned)std::min<int64_t>(z.nch_max, 2048);
        k_compact_count<<<cb, kBlock, 0, s>>>(residual, gr.off, G, w);
        SGC_LAUNCH_CHECK();
        k_chunk_scan<<<1, kScanThreads, 0, s>>>(G, w);
        SGC_LAUNCH_CHECK();
        k_compact_write<<<cb, kBlock, 0, s>>>(residual, gr.off, G, w, out_idx, out_val, cap);
        SGC_LAUNCH_CHECK();
    }
    unsigned sb = (unsigned)std::max<int64_t>(1, std::min<int64_t>(cdiv(L->nseg + 1, kBlock), 1024));
    k_seg_counts<<<sb, kBlock, 0, s>>>(dt->seg_off, L->nseg, out_idx, w, out_counts);
    SGC_LAUNCH_CHECK();
    return SGC_OK;
}
