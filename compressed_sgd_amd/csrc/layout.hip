// layout.hip -- the shared shape table (layout), host helpers, fill kernel.
//
// [SBC] appendix A: both ends of the exchange know every tensor shape, so
// the coded messages carry none; a layout is that shared table.
#include <cmath>
#include <cstring>
#include <new>

#include "sgc_common.h"

namespace sgc {

__global__ void k_fill_u32(uint32_t* p, int64_t count, uint32_t value)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = value;
}

int fill_u32(void* p, int64_t count, uint32_t value, hipStream_t s)
{
    if (count <= 0) return SGC_OK;
    int64_t blocks = cdiv(count, kBlock);
    if (blocks > 4096) blocks = 4096;
    k_fill_u32<<<(unsigned)blocks, kBlock, 0, s>>>((uint32_t*)p, count, value);
    SGC_LAUNCH_CHECK();
    return SGC_OK;
}

int device_tables(sgc_layout* L, DevTables** out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return SGC_EHIP;
    std::lock_guard<std::mutex> lock(L->mu);
    auto it = L->dev.find(dev);
    if (it == L->dev.end()) return SGC_ENOTREADY;
    *out = &it->second;
    return SGC_OK;
}

// The tables of one device: segment offsets and tile prefixes, then the
// global group's {0, n} and {0, tiles}.  Allocated and copied once, at set-up.
static int upload_tables(sgc_layout* L)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return SGC_EHIP;
    std::lock_guard<std::mutex> lock(L->mu);
    if (L->dev.find(dev) != L->dev.end()) return SGC_OK;
    const int64_t ns = L->nseg + 1;
    std::vector<int64_t> host((size_t)(2 * ns + 4));
    std::memcpy(host.data(), L->seg_off.data(), ns * sizeof(int64_t));
    std::memcpy(host.data() + ns, L->seg_tile.data(), ns * sizeof(int64_t));
    host[2 * ns + 0] = 0;
    host[2 * ns + 1] = L->n;
    host[2 * ns + 2] = 0;
    host[2 * ns + 3] = group_tiles(0, L->n);
    DevTables t;
    if (hipMalloc(&t.block, host.size() * sizeof(int64_t)) != hipSuccess) return SGC_EHIP;
    if (hipMemcpy(t.block, host.data(), host.size() * sizeof(int64_t), hipMemcpyHostToDevice) != hipSuccess) {
        (void)hipFree(t.block);
        return SGC_EHIP;
    }
    int64_t* b = (int64_t*)t.block;
    t.seg_off = b;
    t.seg_tile = b + ns;
    t.glob_off = b + 2 * ns;
    t.glob_tile = b + 2 * ns + 2;
    L->dev.emplace(dev, t);
    return SGC_OK;
}

Groups groups_of(sgc_layout* L, const DevTables* d, int32_t scope)
{
    Groups g;
    if (scope == SGC_GLOBAL) {
        g.G = 1;
        g.off = d->glob_off;
        g.tile = d->glob_tile;
        g.ntiles = group_tiles(0, L->n);
    } else {
        g.G = L->nseg;
        g.off = d->seg_off;
        g.tile = d->seg_tile;
        g.ntiles = L->seg_tile[L->nseg];
    }
    return g;
}

std::vector<int64_t> host_group_off(const sgc_layout* L, int32_t scope)
{
    if (scope == SGC_GLOBAL) return {0, L->n};
    return L->seg_off;
}

}  // namespace sgc

using namespace sgc;

extern "C" int sgc_layout_create(const int64_t* seg_numel, int32_t nseg, sgc_layout** out)
{
    if (!out) return SGC_EINVAL;
    *out = nullptr;
    if (!seg_numel || nseg < 1) return SGC_EINVAL;
    int64_t n = 0;
    for (int32_t t = 0; t < nseg; ++t) {
        if (seg_numel[t] < 0) return SGC_EINVAL;
        n += seg_numel[t];
        if (n >= ((int64_t)1 << 31)) return SGC_EINVAL;
    }
    sgc_layout* L = new (std::nothrow) sgc_layout();
    if (!L) return SGC_ENOSPC;
    try {
        L->nseg = nseg;
        L->n = n;
        L->seg_off.resize((size_t)nseg + 1);
        L->seg_tile.resize((size_t)nseg + 1);
        L->seg_off[0] = 0;
        L->seg_tile[0] = 0;
        for (int32_t t = 0; t < nseg; ++t) {
            L->seg_off[t + 1] = L->seg_off[t] + seg_numel[t];
            L->seg_tile[t + 1] = L->seg_tile[t] + group_tiles(L->seg_off[t], L->seg_off[t + 1]);
        }
    } catch (...) {
        delete L;
        return SGC_ENOSPC;
    }
    *out = L;
    return SGC_OK;
}

extern "C" int sgc_layout_upload(sgc_layout* L)
{
    if (!L) return SGC_EINVAL;
    const int rc = upload_tables(L);
    if (rc) return rc;
    // The no-allocation entry point's scratch address on this device.  A
    // failure here is not the layout's: sgc_compress_noalloc reports it.
    (void)scratch_init();
    return SGC_OK;
}

extern "C" void sgc_layout_destroy(sgc_layout* L)
{
    if (!L) return;
    for (auto& kv : L->dev) {
        int cur = 0;
        if (hipGetDevice(&cur) == hipSuccess && hipSetDevice(kv.first) == hipSuccess) {
            (void)hipFree(kv.second.block);
            (void)hipSetDevice(cur);
        }
    }
    delete L;
}

extern "C" int64_t sgc_layout_numel(const sgc_layout* L) { return L ? L->n : -1; }
extern "C" int32_t sgc_layout_nseg(const sgc_layout* L) { return L ? L->nseg : -1; }

extern "C" int64_t sgc_keep_count(int64_t n, uint32_t keep_ppm)
{
    if (n < 0 || n >= ((int64_t)1 << 31) || keep_ppm > 1000000) return -1;
    return keep_count(n, keep_ppm);
}

// Mean Rice code length of geometric gaps at density p ([SBC] §II Optimal
// Position Encoding): b + 1/(1 - (1-p)^(2^b)).
static double rice_mean_bits(int b, double p) { return b + 1.0 / (1.0 - std::pow(1.0 - p, std::ldexp(1.0, b))); }

extern "C" int32_t sgc_rice_param(double p)
{
    if (!(p > 0.0 && p <= 1.0)) return -1;
    int32_t best = 0;
    double bits = rice_mean_bits(0, p);
    for (int b = 1; b <= 30; ++b) {
        double e = rice_mean_bits(b, p);
        if (e < bits) { bits = e; best = b; }
    }
    return best;
}

// Warm-up schedule ([SBC] appendix A, Warm-up Training: the kept fraction
// falls exponentially, from 25% to 0.1%, over the first epochs): the kept
// parts per million of step `step` of a `steps`-step warm-up,
// start * (end / start)^(step / (steps - 1)) rounded to the nearest integer;
// `start` at step 0, `end` from step steps - 1 on.
extern "C" int64_t sgc_warmup_ppm(int64_t step, int64_t steps, uint32_t start_ppm, uint32_t end_ppm)
{
    if (step < 0 || steps < 1 || start_ppm == 0 || end_ppm == 0 || start_ppm > 1000000 || end_ppm > 1000000)
        return -1;
    if (steps == 1 || step >= steps - 1) return end_ppm;
    if (step == 0) return start_ppm;
    const double u = (double)step / (double)(steps - 1);
    const double p = (double)start_ppm * std::pow((double)end_ppm / (double)start_ppm, u);
    return (int64_t)std::floor(p + 0.5);
}

extern "C" const char* sgc_strerror(int code)
{
    switch (code) {
    case SGC_OK: return "ok";
    case SGC_EINVAL: return "invalid argument";
    case SGC_ENOSPC: return "workspace or output capacity too small";
    case SGC_EHIP: return "HIP runtime or launch failure";
    case SGC_EUNSUPPORTED: return "unsupported combination";
    case SGC_ENOTREADY: return "layout not uploaded to the current device (sgc_layout_upload)";
    default: return "unknown error";
    }
}

extern "C" int32_t sgc_abi_version(void) { return SGC_ABI_VERSION; }
