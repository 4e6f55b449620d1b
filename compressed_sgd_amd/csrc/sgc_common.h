// sgc_common.h -- internals shared by the HIP sources of libsgc (gfx950).
//
// Citations (page title, then section):
//   [AH17]  "Sparse Communication for Distributed Gradient Descent" (Aji & Heafield)
//   [AHB19] "Combining Global Sparse Gradients with Local Gradients in Distributed
//           Neural Network Training" (Aji, Heafield & Bogoychev)
//   [SBC]   "Sparse Binary Compression: Towards Distributed Deep Learning with
//           minimal Communication" (Sattler et al.)
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <map>
#include <mutex>
#include <vector>

#include "../../include/sgc.h"

namespace sgc {

// ---------------------------------------------------------------- geometry
// Pass-1 tile: 4096 elements, 512 threads x 2 float4 slots (measured on
// gfx950: about 1% faster than 256 x 4, while 1024 x 1, 256 x 8 and
// 8192-element tiles are slower, and smaller tiles lose more to their
// per-tile work than they gain).  Tiles never
// straddle a selection group; inside a group they sit on a 4-element-aligned
// grid so that every full slot is one aligned 16-byte access.
constexpr int kBlock = 256;
constexpr int kPassThreads = 512;
constexpr int64_t kTile = 4096;
// Candidate slots per tile region: a power of two from kTileCapMin up to a
// whole tile, chosen per call as about 1.5 times the expected candidates of
// a tile (the kept fraction plus the probe's band) -- a power-of-two region
// stride keeps pass 1's region writes at full speed.  A tile with more
// candidates than its region is redone from the residual (which holds acc
// there after pass 1).
constexpr int kTileCapMin = 256;
inline int64_t region_capacity(uint32_t ppm)
{
    const double expect = (double)kTile * (double)ppm / 1e6 * 1.15;
    int64_t cap = kTileCapMin;
    while (cap < kTile && (double)cap < 1.5 * expect + 64.0) cap *= 2;
    return cap;
}
// Chunk of the selection / compaction kernels: 256 threads x 16 contiguous.
constexpr int kPer = 16;
constexpr int64_t kChunk = (int64_t)kBlock * kPer;  // 4096 entries
// Radix digits of the 31-bit magnitude key: bits 30..20, 19..10, 9..0.
constexpr int kBins = 2048;
// Rice encoder block: codes per encode block, and look-ahead codes.
constexpr int64_t kEncCodes = 2048;
constexpr int kEncAhead = 32;
// Dense output tile of decode-accumulate.
constexpr int64_t kOutTile = 8192;
constexpr int kOutTileLog = 13;
static_assert(kOutTile == (int64_t)1 << kOutTileLog, "output tile size");

constexpr uint32_t kNoKey = 0x80000000u;  // above every 31-bit magnitude key

// ------------------------------------------------------- shared arithmetic
// Magnitude key: for finite floats the order of |x| is the order of the
// unsigned integer formed by the low 31 bits (+0 and -0 share key 0).
__host__ __device__ inline uint32_t mag_key(float x)
{
    union { float f; uint32_t u; } c;
    c.f = x;
    return c.u & 0x7fffffffu;
}

// k = ceil(m * ppm / 1e6), at most m ([AH17] Abstract; [SBC] §II Sparse
// Binarization).  m < 2^31 and ppm <= 1e6 keep the product below 2^51.
__host__ __device__ inline int64_t keep_count(int64_t m, uint32_t ppm)
{
    if (m <= 0) return 0;
    int64_t k = (m * (int64_t)ppm + 999999) / 1000000;
    return k < m ? k : m;
}

// Sample size of the sampled-threshold mode.
__host__ __device__ inline int64_t sampled_count(int64_t m, uint32_t div, uint32_t smin)
{
    if (m <= 0) return 0;
    int64_t s = (m + (int64_t)div - 1) / (int64_t)div;
    if (s < (int64_t)smin) s = smin;
    return s < m ? s : m;
}

// Probe of the exact mode: it only places the candidate bounds, the result
// never depends on it.  Runs of kRun contiguous elements (one 64-byte
// sector each) at systematic positions; a small group is read whole.
constexpr int kRun = 16;
__host__ __device__ inline int64_t probe_points(int64_t m)  // 0: read the whole group
{
    if (m <= (int64_t)kRun * 64) return 0;
    int64_t p = m / 4096;
    if (p < 64) p = 64;
    if (p > 16384) p = 16384;
    return p;
}
__host__ __device__ inline int64_t probe_count(int64_t m)
{
    const int64_t p = probe_points(m);
    return p ? p * kRun : (m > 0 ? m : 0);
}

// Pass-1 tiles of a group [lo, hi): aligned grid starting at lo & ~3.
__host__ __device__ inline int64_t group_tiles(int64_t lo, int64_t hi)
{
    if (hi <= lo) return 0;
    int64_t a = lo & ~(int64_t)3;
    return (hi - a + kTile - 1) / kTile;
}

__host__ __device__ inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Largest i in [0, len) with a[i] <= x, for ascending a with a[0] <= x.
template <typename T>
__device__ inline int64_t find_bucket(const T* a, int64_t len, T x)
{
    int64_t lo = 0, hi = len - 1;
    while (lo < hi) {
        int64_t mid = (lo + hi + 1) >> 1;
        if (a[mid] <= x) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// --------------------------------------------------------- block helpers
// Exclusive scan of one value per thread over a 256-thread block.  `tmp`
// is shared scratch of kBlock/64 + 1 entries.  Returns the exclusive prefix
// and writes the block total to *total.  Every thread must call it.
template <typename T>
__device__ inline T block_exclusive_scan(T v, T* tmp, T* total)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    T x = v;
    // inclusive scan inside the wave
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        T y = __shfl_up(x, d, 64);
        if (lane >= d) x += y;
    }
    if (lane == 63) tmp[wave] = x;
    __syncthreads();
    if (threadIdx.x == 0) {
        T run = 0;
        for (int w = 0; w < kBlock / 64; ++w) { T t = tmp[w]; tmp[w] = run; run += t; }
        tmp[kBlock / 64] = run;
    }
    __syncthreads();
    T res = tmp[wave] + x - v;
    *total = tmp[kBlock / 64];
    __syncthreads();
    return res;
}

// Exclusive scan over a workgroup of NTH threads (a multiple of 64, at most
// 1024); tmp holds NTH/64 + 1 entries.  Every thread gets its exclusive
// prefix and the total; the trailing barrier lets the caller reuse tmp.
template <int NTH, typename T>
__device__ inline T block_scan_excl(T v, T* tmp, T* total)
{
    static_assert(NTH % 64 == 0 && NTH <= 1024, "whole waves");
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
        for (int w = 0; w < NTH / 64; ++w) { T t = tmp[w]; tmp[w] = run; run += t; }
        tmp[NTH / 64] = run;
    }
    __syncthreads();
    T res = tmp[wave] + x - v;
    *total = tmp[NTH / 64];
    __syncthreads();
    return res;
}

// ------------------------------------------------------------- layout
struct DevTables {
    int64_t* seg_off = nullptr;   // [nseg+1]
    int64_t* seg_tile = nullptr;  // [nseg+1] pass-1 tile prefix per segment
    int64_t* glob_off = nullptr;  // [2] = {0, n}
    int64_t* glob_tile = nullptr; // [2] = {0, tiles of [0, n)}
    void* block = nullptr;
};

}  // namespace sgc

struct sgc_layout {
    int32_t nseg = 0;
    int64_t n = 0;
    std::vector<int64_t> seg_off;   // [nseg+1]
    std::vector<int64_t> seg_tile;  // [nseg+1]
    std::mutex mu;
    std::map<int, sgc::DevTables> dev;
};

namespace sgc {

// Selection groups of a scope: GLOBAL -> {[0, n)}, PER_SEGMENT -> segments.
struct Groups {
    int32_t G;
    const int64_t* off;   // device [G+1]
    const int64_t* tile;  // device [G+1]
    int64_t ntiles;       // host
};

int device_tables(sgc_layout* L, DevTables** out);
Groups groups_of(sgc_layout* L, const DevTables* d, int32_t scope);
std::vector<int64_t> host_group_off(const sgc_layout* L, int32_t scope);

// Workspace carving: the same sequence of take() calls sizes the workspace
// (base == nullptr) and assigns the pointers.
struct Carver {
    char* base;
    size_t off = 0;
    explicit Carver(void* b) : base((char*)b) {}
    template <typename T>
    T* take(int64_t count)
    {
        off = (off + 255) & ~(size_t)255;
        T* p = base ? (T*)(base + off) : nullptr;
        off += (size_t)(count > 0 ? count : 1) * sizeof(T);
        return p;
    }
};

inline int hip_ok(hipError_t e) { return e == hipSuccess ? SGC_OK : SGC_EHIP; }
#define SGC_LAUNCH_CHECK()                                   \
    do {                                                     \
        if (hipGetLastError() != hipSuccess) return SGC_EHIP; \
    } while (0)

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Zero `count` 32-bit words with a kernel (no memset nodes in a stream that
// may be captured into a graph).
int fill_u32(void* p, int64_t count, uint32_t value, hipStream_t s);

// sgc_compress with the stream already cast (shared with the no-allocation
// entry point, which passes the library's own scratch buffer as ws).
int compress_call(const sgc_layout* L, const sgc_compress_opts* o, const float* grad, float* residual,
                  int32_t* out_idx, float* out_val, int64_t cap, int64_t* out_counts, uint32_t* dstatus, void* ws,
                  size_t ws_bytes, hipStream_t stream);

// The device address of the no-allocation scratch buffer on the current
// device: looked up once per device by scratch_init (called from the
// layout upload, the library's per-device set-up); scratch_device returns
// nullptr where that has not happened or failed.
int scratch_init();
void* scratch_device();

}  // namespace sgc
