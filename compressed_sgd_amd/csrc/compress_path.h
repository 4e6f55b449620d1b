// compress_path.h -- what the two compress pipelines share, and how the
// entry points (compress.hip) call them.
//
// Both pipelines compute the same result bit for bit ([SBC] §II Residual
// Accumulation and Sparse Binarization; [AH17] Abstract): they differ only
// in how the exact selection finds its threshold after the one pass over the
// gradient.
//  * gather (compress_gather.hip): every candidate of a group (|acc| above a
//    probe-estimated lower bound) is copied into one ordered candidate array,
//    which is radix-selected and compacted.  Its fixed cost after the pass is
//    small, so it is the faster one at low kept fractions.
//  * window (compress_window.hip): the probe also gives an upper bound above
//    which every entry is surely kept; only the entries between the bounds
//    are radix-selected, from short per-tile lists, and the kept entries are
//    written straight from the per-tile candidate regions.  It moves far
//    fewer bytes than gather when many entries are kept.
#pragma once

#include "sgc_common.h"

namespace sgc {

// Momentum correction of one compress call ([SBC] appendix A): off, or on
// with coefficient beta and the momentum vector u (u <- beta*u + g is what
// goes into the residual; u <- +0 where an entry is sent).
struct NoMom {
    static constexpr bool on = false;
    float beta;
    float* u;
};
struct Mom {
    static constexpr bool on = true;
    float beta;
    float* u;
};

// u' = fp32(fp32(beta * u) + g), two roundings (the build disables contraction)
__device__ inline float mom_update(float beta, float u, float g)
{
    const float bu = beta * u;
    return bu + g;
}

// One compress call, arguments checked by the entry point: o is EXACT or
// SAMPLED (the SGC_HOLD_KEPT flag taken out into hold), cap covers the exact
// keep counts, grad/residual/u are 16-byte aligned.
struct CompressCall {
    sgc_layout* L;
    sgc_compress_opts o;
    bool hold;
    bool mom;
    float beta;
    float* u;
    const float* grad;
    float* residual;
    int32_t* out_idx;
    float* out_val;
    int64_t cap;
    int64_t* out_counts;
    uint32_t* dstatus;
    void* ws;
    size_t ws_bytes;
    hipStream_t s;
};

namespace gather {
size_t workspace_bytes(const sgc_layout* L, const sgc_compress_opts* o, bool mom);
int run(const CompressCall& c);
}  // namespace gather

namespace window {
size_t workspace_bytes(const sgc_layout* L, const sgc_compress_opts* o, bool mom);
int run(const CompressCall& c);
}  // namespace window

// Measurement hook: events recorded around the fused pass (benchmarks only).
extern hipEvent_t g_pass_start, g_pass_stop;

}  // namespace sgc
