// compress.hip -- the compress entry points (sgc_compress, sgc_compress_momentum
// and their workspace queries): argument checks, the accumulate-only step,
// and the choice between the two selection pipelines.
//
// Method ([SBC] §II Residual Accumulation and Sparse Binarization; [AH17]
// Abstract): acc = fp32(residual + grad); keep the largest-|acc| fraction of
// each selection group; send (index, value) ascending; the residual keeps
// everything else.  [SBC] §II Communication Delay: between exchanges only
// residual += grad is done (SGC_ACCUMULATE_ONLY).
//
// Both pipelines give the same result bit for bit.  Measured on MI355X:
// above a kept fraction of about 2.5% (candidate regions larger than 256
// slots) window is ahead at every size (2^30 elements: 2.58 against 2.90 ms
// at 5%, 3.7 against 5.7 ms at 25%); below it gather is ahead on vectors of
// up to 10^8 elements (its fixed cost after the pass over the gradient is
// lower), the two are level at 2^28 and 2^29, and window is ahead at 2^30
// (2.29 against 2.34 ms at 1%).  SGC_PATH_GATHER / SGC_PATH_WINDOW force one.
#include "compress_path.h"

#include <cmath>

namespace sgc {

hipEvent_t g_pass_start = nullptr, g_pass_stop = nullptr;

typedef float f4 __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------ accumulate
// SGC_ACCUMULATE_ONLY: r <- r + g over the whole vector (float4 body, the
// last n % 4 elements by workgroup 0).  With momentum: u <- beta*u + g first,
// and r <- r + u.
template <typename M>
__global__ __launch_bounds__(kBlock) void k_accumulate(const float* __restrict__ g, float* __restrict__ r, int64_t n,
                                                      M m)
{
    const int64_t n4 = n >> 2;
    const f4* g4 = (const f4*)g;
    f4* r4 = (f4*)r;
    const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (i < n4) {
        f4 a = __builtin_nontemporal_load(r4 + i);
        f4 b = __builtin_nontemporal_load(g4 + i);
        if constexpr (M::on) {
            f4* u4 = (f4*)m.u;
            const f4 uo = __builtin_nontemporal_load(u4 + i);
            f4 up;
#pragma unroll
            for (int j = 0; j < 4; ++j) up[j] = mom_update(m.beta, uo[j], b[j]);
            __builtin_nontemporal_store(up, u4 + i);
            b = up;
        }
        __builtin_nontemporal_store(a + b, r4 + i);
    }
    if (blockIdx.x == 0 && threadIdx.x < (n & 3)) {
        const int64_t j = (n4 << 2) + threadIdx.x;
        float gj = g[j];
        if constexpr (M::on) {
            gj = mom_update(m.beta, m.u[j], gj);
            m.u[j] = gj;
        }
        r[j] = r[j] + gj;
    }
}

template <typename M>
static int accumulate(const sgc_layout* L, const float* grad, float* residual, M m, hipStream_t s)
{
    if (L->n == 0) return SGC_OK;
    const int64_t blocks = cdiv(std::max<int64_t>(L->n >> 2, 1), kBlock);
    k_accumulate<M><<<(unsigned)blocks, kBlock, 0, s>>>(grad, residual, L->n, m);
    SGC_LAUNCH_CHECK();
    return SGC_OK;
}

// The selection mode without the SGC_HOLD_KEPT flag.
static int32_t base_mode(const sgc_compress_opts* o) { return o->mode & ~(int32_t)SGC_HOLD_KEPT; }

static bool opts_ok(const sgc_layout* L, const sgc_compress_opts* o)
{
    if (!L || !o) return false;
    const int32_t bm = base_mode(o);
    if (bm != SGC_EXACT && bm != SGC_SAMPLED && bm != SGC_ACCUMULATE_ONLY) return false;
    if ((o->mode & SGC_HOLD_KEPT) && bm == SGC_ACCUMULATE_ONLY) return false;
    if (o->scope != SGC_GLOBAL && o->scope != SGC_PER_SEGMENT) return false;
    if (o->keep_ppm > 1000000) return false;
    if (bm == SGC_SAMPLED && o->sample_div == 0) return false;
    if (o->path != SGC_PATH_AUTO && o->path != SGC_PATH_GATHER && o->path != SGC_PATH_WINDOW) return false;
    return true;
}

// Vectors from this size on take the window pipeline at any kept fraction.
constexpr int64_t kWindowMinN = (int64_t)1 << 29;

// The options with the flag taken out of the mode (the pipelines take it as
// CompressCall::hold) and the pipeline decided.
static sgc_compress_opts plain_opts(const sgc_layout* L, const sgc_compress_opts* o)
{
    sgc_compress_opts p = *o;
    p.mode = base_mode(o);
    if (p.path == SGC_PATH_AUTO)
        p.path = (region_capacity(p.keep_ppm) > kTileCapMin || L->n >= kWindowMinN) ? SGC_PATH_WINDOW
                                                                                    : SGC_PATH_GATHER;
    return p;
}

static size_t path_workspace(const sgc_layout* L, const sgc_compress_opts* p, bool mom)
{
    return p->path == SGC_PATH_WINDOW ? window::workspace_bytes(L, p, mom) : gather::workspace_bytes(L, p, mom);
}

// Checks shared by both entry points, then the chosen pipeline.
static int select_call(CompressCall& a)
{
    const sgc_compress_opts* o = &a.o;
    if (!a.out_counts || a.cap < 0 || a.cap >= ((int64_t)1 << 31)) return SGC_EINVAL;
    if (a.cap > 0 && (!a.out_idx || !a.out_val)) return SGC_EINVAL;
    if (o->mode == SGC_EXACT) {
        std::vector<int64_t> hoff = host_group_off(a.L, o->scope);
        int64_t K = 0;
        for (size_t g = 0; g + 1 < hoff.size(); ++g) K += keep_count(hoff[g + 1] - hoff[g], o->keep_ppm);
        if (a.cap < K) return SGC_EINVAL;
    }
    return o->path == SGC_PATH_WINDOW ? window::run(a) : gather::run(a);
}

int compress_call(const sgc_layout* Lc, const sgc_compress_opts* o, const float* grad, float* residual,
                  int32_t* out_idx, float* out_val, int64_t cap, int64_t* out_counts, uint32_t* dstatus, void* ws,
                  size_t ws_bytes, hipStream_t stream)
{
    sgc_layout* L = const_cast<sgc_layout*>(Lc);
    if (!opts_ok(L, o)) return SGC_EINVAL;
    if ((L->n > 0 && (!grad || !residual)) || !aligned16(grad) || !aligned16(residual)) return SGC_EINVAL;
    const sgc_compress_opts p = plain_opts(L, o);
    if (p.mode == SGC_ACCUMULATE_ONLY) return accumulate(L, grad, residual, NoMom{0.0f, nullptr}, stream);
    CompressCall a{L,       p,   (o->mode & SGC_HOLD_KEPT) != 0, false, 0.0f, nullptr, grad, residual, out_idx,
                   out_val, cap, out_counts, dstatus, ws, ws_bytes, stream};
    return select_call(a);
}

}  // namespace sgc

using namespace sgc;

extern "C" int sgc_set_pass_events(void* start, void* stop)
{
    if ((start == nullptr) != (stop == nullptr)) return SGC_EINVAL;
    g_pass_start = (hipEvent_t)start;
    g_pass_stop = (hipEvent_t)stop;
    return SGC_OK;
}

extern "C" size_t sgc_compress_workspace(const sgc_layout* L, const sgc_compress_opts* o, int64_t cap)
{
    if (!opts_ok(L, o) || cap < 0) return 0;
    const sgc_compress_opts p = plain_opts(L, o);
    if (p.mode == SGC_ACCUMULATE_ONLY) return 0;
    return path_workspace(L, &p, false);
}

extern "C" size_t sgc_compress_momentum_workspace(const sgc_layout* L, const sgc_compress_opts* o, int64_t cap)
{
    if (!opts_ok(L, o) || cap < 0 || (o->mode & SGC_HOLD_KEPT)) return 0;
    const sgc_compress_opts p = plain_opts(L, o);
    if (p.mode == SGC_ACCUMULATE_ONLY) return 0;
    return path_workspace(L, &p, true);
}

extern "C" int sgc_compress(const sgc_layout* Lc, const sgc_compress_opts* o, const float* grad, float* residual,
                            int32_t* out_idx, float* out_val, int64_t cap, int64_t* out_counts, uint32_t* dstatus,
                            void* ws, size_t ws_bytes, sgc_stream_t stream)
{
    return compress_call(Lc, o, grad, residual, out_idx, out_val, cap, out_counts, dstatus, ws, ws_bytes,
                         (hipStream_t)stream);
}

extern "C" int sgc_compress_momentum(const sgc_layout* Lc, const sgc_compress_opts* o, float beta, const float* grad,
                                     float* momentum, float* residual, int32_t* out_idx, float* out_val, int64_t cap,
                                     int64_t* out_counts, uint32_t* dstatus, void* ws, size_t ws_bytes,
                                     sgc_stream_t stream)
{
    sgc_layout* L = const_cast<sgc_layout*>(Lc);
    if (!opts_ok(L, o) || !std::isfinite(beta)) return SGC_EINVAL;
    if (o->mode & SGC_HOLD_KEPT) return SGC_EUNSUPPORTED;  // momentum masking writes the sent entries anyway
    if ((L->n > 0 && (!grad || !residual || !momentum)) || !aligned16(grad) || !aligned16(residual) ||
        !aligned16(momentum))
        return SGC_EINVAL;
    const sgc_compress_opts p = plain_opts(L, o);
    if (p.mode == SGC_ACCUMULATE_ONLY)
        return accumulate(L, grad, residual, Mom{beta, momentum}, (hipStream_t)stream);
    CompressCall a{L,       p,   false,      true,    beta, momentum, grad,     residual, out_idx,
                   out_val, cap, out_counts, dstatus, ws,   ws_bytes, (hipStream_t)stream};
    return select_call(a);
}
