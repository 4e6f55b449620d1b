// noalloc.hip -- sgc_compress_noalloc: the compress step with the library's
// own scratch buffer, for callers that cannot allocate device memory.
//
// The scratch buffer is a file-scope __device__ array: every GPU the
// library runs on holds its own copy, at its own address, from the moment
// this code object is loaded there until the process ends.  In host code the
// array's name stands for a host-side shadow, not for device memory: its
// device address is looked up once per device (hipGetSymbolAddress, with that
// device current) and only that address is ever handed to kernels.
#include "sgc_common.h"

namespace sgc {

constexpr size_t kScratchBytes = SGC_NOALLOC_SCRATCH_BYTES;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

static std::mutex g_scratch_mu;
static std::map<int, void*> g_scratch_ptr;  // device -> device address of scratch

int scratch_init()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return SGC_EHIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr.count(dev)) return SGC_OK;
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
        (void)hipGetLastError();  // leave no sticky error for the caller's next call
        return SGC_EHIP;
    }
    g_scratch_ptr[dev] = ptr;
    return SGC_OK;
}

void* scratch_device()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    auto it = g_scratch_ptr.find(dev);
    return it == g_scratch_ptr.end() ? nullptr : it->second;
}

}  // namespace sgc

using namespace sgc;

extern "C" int sgc_compress_noalloc(const sgc_layout* L, const sgc_compress_opts* o, const float* grad,
                                    float* residual, int32_t* out_idx, float* out_val, int64_t cap,
                                    int64_t* out_counts, uint32_t* dstatus, sgc_stream_t stream)
{
    if (!L || !o) return SGC_EINVAL;
    if ((o->mode & ~(int32_t)SGC_HOLD_KEPT) == SGC_ACCUMULATE_ONLY)  // needs no workspace
        return compress_call(L, o, grad, residual, out_idx, out_val, cap, out_counts, dstatus, nullptr, 0,
                             (hipStream_t)stream);
    const size_t need = sgc_compress_workspace(L, o, cap);
    if (need == 0) return SGC_EINVAL;              // bad options or capacity
    if (need > kScratchBytes) return SGC_ENOSPC;   // beyond the scratch buffer
    void* ws = scratch_device();
    if (!ws) return SGC_ENOTREADY;                 // no layout upload on this device (or it failed there)
    return compress_call(L, o, grad, residual, out_idx, out_val, cap, out_counts, dstatus, ws, kScratchBytes,
                         (hipStream_t)stream);
}
