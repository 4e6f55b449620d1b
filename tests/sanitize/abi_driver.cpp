// Drives the host side of every entry point of libsgc without a GPU: layout
// creation and destruction, the host helpers, the workspace and bound
// queries, and every argument error the compute calls report before they
// queue GPU work.  Built with -fsanitize=address,undefined on the host code
// of the library, so the validation paths run under the sanitizers.  Exit
// status 0 when every return code is the documented one.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <vector>

#include "sgc.h"

static int failures = 0;
#define CHECK(c)                                                               \
    do {                                                                       \
        if (!(c)) {                                                            \
            std::fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); \
            ++failures;                                                        \
        }                                                                      \
    } while (0)

int main()
{
    // stand-in device pointers: never dereferenced, validation fails first
    void* A = reinterpret_cast<void*>(uintptr_t(4096));
    void* MIS = reinterpret_cast<void*>(uintptr_t(4100));
    float* Af = static_cast<float*>(A);
    int32_t* Ai = static_cast<int32_t*>(A);
    int64_t* Al = static_cast<int64_t*>(A);
    uint32_t* Au = static_cast<uint32_t*>(A);
    uint64_t* Aq = static_cast<uint64_t*>(A);

    CHECK(sgc_abi_version() == SGC_ABI_VERSION);
    for (int c = 1; c >= -6; --c) CHECK(sgc_strerror(c) != nullptr);
    CHECK(sgc_keep_count(1 << 20, 10000) == 10486);
    CHECK(sgc_keep_count(-1, 10) == -1 && sgc_keep_count(10, 1000001) == -1);
    CHECK(sgc_keep_count((int64_t(1) << 31) - 1, 1000000) == (int64_t(1) << 31) - 1);
    CHECK(sgc_rice_param(0.01) == 6 && sgc_rice_param(0.0) == -1 && sgc_rice_param(NAN) == -1);
    CHECK(sgc_warmup_ppm(1, 6, 250000, 1000) == 82861 && sgc_warmup_ppm(0, 0, 1, 1) == -1);

    sgc_layout* L = nullptr;
    const int64_t bad[3] = {5, -1, 3};
    CHECK(sgc_layout_create(bad, 3, &L) == SGC_EINVAL && L == nullptr);
    CHECK(sgc_layout_create(bad, 0, &L) == SGC_EINVAL);
    CHECK(sgc_layout_create(nullptr, 1, &L) == SGC_EINVAL);
    CHECK(sgc_layout_create(bad, 1, nullptr) == SGC_EINVAL);
    const int64_t big[2] = {int64_t(1) << 30, int64_t(1) << 30};
    CHECK(sgc_layout_create(big, 2, &L) == SGC_EINVAL);
    const int64_t edge[2] = {int64_t(1) << 30, (int64_t(1) << 30) - 1};
    CHECK(sgc_layout_create(edge, 2, &L) == SGC_OK);
    CHECK(sgc_layout_numel(L) == (int64_t(1) << 31) - 1 && sgc_layout_nseg(L) == 2);
    sgc_layout_destroy(L);
    sgc_layout_destroy(nullptr);
    CHECK(sgc_layout_numel(nullptr) == -1 && sgc_layout_nseg(nullptr) == -1);
    CHECK(sgc_layout_upload(nullptr) == SGC_EINVAL);

    std::vector<int64_t> sizes = {1000, 24, 0, 5000};
    CHECK(sgc_layout_create(sizes.data(), (int32_t)sizes.size(), &L) == SGC_OK);
    const int64_t n = sgc_layout_numel(L);
    const int64_t k = sgc_keep_count(n, 10000);
    sgc_compress_opts o = {SGC_EXACT, SGC_GLOBAL, 10000, 1000, 65536};
    const size_t need = sgc_compress_workspace(L, &o, k);
    CHECK(need > 0);
    CHECK(sgc_compress(L, nullptr, Af, Af, Ai, Af, k, Al, nullptr, A, need, nullptr) == SGC_EINVAL);
    sgc_compress_opts badm = {7, 0, 10000, 1000, 1}, bads = {0, 5, 10000, 1000, 1}, badp = {0, 0, 1000001, 1000, 1},
                      badd = {1, 0, 10000, 0, 1};
    for (auto* b : {&badm, &bads, &badp, &badd}) {
        CHECK(sgc_compress(L, b, Af, Af, Ai, Af, k, Al, nullptr, A, need, nullptr) == SGC_EINVAL);
        CHECK(sgc_compress_workspace(L, b, k) == 0);
        CHECK(sgc_compress_noalloc(L, b, Af, Af, Ai, Af, k, Al, nullptr, nullptr) == SGC_EINVAL);
    }
    CHECK(sgc_compress(L, &o, nullptr, Af, Ai, Af, k, Al, nullptr, A, need, nullptr) == SGC_EINVAL);
    CHECK(sgc_compress(L, &o, Af, (float*)MIS, Ai, Af, k, Al, nullptr, A, need, nullptr) == SGC_EINVAL);
    CHECK(sgc_compress(L, &o, Af, Af, Ai, Af, k - 1, Al, nullptr, A, need, nullptr) == SGC_EINVAL);
    CHECK(sgc_compress(L, &o, Af, Af, Ai, Af, k, nullptr, nullptr, A, need, nullptr) == SGC_EINVAL);
    CHECK(sgc_compress(L, &o, Af, Af, nullptr, Af, k, Al, nullptr, A, need, nullptr) == SGC_EINVAL);
    CHECK(sgc_compress(L, &o, Af, Af, Ai, Af, k, Al, nullptr, nullptr, need, nullptr) == SGC_ENOSPC);
    CHECK(sgc_compress(L, &o, Af, Af, Ai, Af, k, Al, nullptr, A, need - 1, nullptr) == SGC_ENOSPC);
    CHECK(sgc_compress(nullptr, &o, Af, Af, Ai, Af, k, Al, nullptr, A, need, nullptr) == SGC_EINVAL);
    CHECK(sgc_compress_noalloc(nullptr, &o, Af, Af, Ai, Af, k, Al, nullptr, nullptr) == SGC_EINVAL);
    sgc_compress_opts held = {SGC_EXACT | SGC_HOLD_KEPT, SGC_GLOBAL, 10000, 1000, 65536};
    sgc_compress_opts acch = {SGC_ACCUMULATE_ONLY | SGC_HOLD_KEPT, SGC_GLOBAL, 10000, 1000, 65536};
    CHECK(sgc_compress_workspace(L, &held, k) == need);
    CHECK(sgc_compress(L, &acch, Af, Af, Ai, Af, k, Al, nullptr, A, need, nullptr) == SGC_EINVAL);

    const size_t mneed = sgc_compress_momentum_workspace(L, &o, k);
    CHECK(mneed > need);
    CHECK(sgc_compress_momentum(L, &o, NAN, Af, Af, Af, Ai, Af, k, Al, nullptr, A, mneed, nullptr) == SGC_EINVAL);
    CHECK(sgc_compress_momentum(L, &o, INFINITY, Af, Af, Af, Ai, Af, k, Al, nullptr, A, mneed, nullptr) ==
          SGC_EINVAL);
    CHECK(sgc_compress_momentum(L, &o, 0.9f, Af, nullptr, Af, Ai, Af, k, Al, nullptr, A, mneed, nullptr) ==
          SGC_EINVAL);
    CHECK(sgc_compress_momentum(L, &o, 0.9f, Af, (float*)MIS, Af, Ai, Af, k, Al, nullptr, A, mneed, nullptr) ==
          SGC_EINVAL);
    CHECK(sgc_compress_momentum(L, &o, 0.9f, Af, Af, Af, Ai, Af, k, Al, nullptr, A, mneed - 1, nullptr) ==
          SGC_ENOSPC);
    CHECK(sgc_compress_momentum(L, &held, 0.9f, Af, Af, Af, Ai, Af, k, Al, nullptr, A, mneed, nullptr) ==
          SGC_EUNSUPPORTED);

    const size_t bneed = sgc_binarize_workspace(L, 10);
    CHECK(bneed > 0 && sgc_binarize_workspace(nullptr, 10) == 0 && sgc_binarize_workspace(L, -1) == 0);
    CHECK(sgc_binarize(L, 3, Ai, Af, Al, 10, Af, Ai, Al, Af, Au, A, bneed, nullptr) == SGC_EINVAL);
    CHECK(sgc_binarize(L, 2 | SGC_BIN_HELD, Ai, Af, Al, 10, Af, Ai, Al, Af, Au, A, bneed, nullptr) == SGC_EINVAL);
    CHECK(sgc_binarize(L, SGC_BIN_SBC, Ai, Af, Al, -1, Af, Ai, Al, Af, Au, A, bneed, nullptr) == SGC_EINVAL);
    CHECK(sgc_binarize(L, SGC_BIN_SBC, Ai, Af, nullptr, 10, Af, Ai, Al, Af, Au, A, bneed, nullptr) == SGC_EINVAL);
    CHECK(sgc_binarize(L, SGC_BIN_SBC, Ai, Af, Al, 10, nullptr, Ai, Al, Af, Au, A, bneed, nullptr) == SGC_EINVAL);
    CHECK(sgc_binarize(L, SGC_BIN_SBC, Ai, Af, Al, 10, Af, nullptr, Al, Af, Au, A, bneed, nullptr) == SGC_EINVAL);
    CHECK(sgc_binarize(L, SGC_BIN_2BIT, Ai, Af, Al, 10, Af, Ai, Al, Af, nullptr, A, bneed, nullptr) == SGC_EINVAL);
    CHECK(sgc_binarize(L, SGC_BIN_SBC, Ai, Af, Al, 10, Af, Ai, Al, Af, Au, nullptr, bneed, nullptr) == SGC_ENOSPC);
    CHECK(sgc_binarize(L, SGC_BIN_SBC, Ai, Af, Al, 10, Af, Ai, Al, Af, Au, A, bneed - 1, nullptr) == SGC_ENOSPC);

    const int64_t cap = 100;
    const int64_t wb = sgc_encode_word_bound(L, SGC_GLOBAL, 6, cap);
    const int64_t cb = sgc_encode_chunk_bound(L, SGC_PER_SEGMENT, cap);
    CHECK(wb > 0 && cb > 0);
    CHECK(sgc_encode_word_bound(L, SGC_GLOBAL, 31, cap) == -1 && sgc_encode_word_bound(L, 7, 6, cap) == -1);
    const size_t eneed = sgc_encode_workspace(L, SGC_GLOBAL, cap);
    CHECK(eneed > 0);
    CHECK(sgc_encode(L, 2, 6, Ai, Al, cap, Au, wb, Aq, Aq, Aq, cb, nullptr, A, eneed, nullptr) == SGC_EINVAL);
    CHECK(sgc_encode(L, 0, -1, Ai, Al, cap, Au, wb, Aq, Aq, Aq, cb, nullptr, A, eneed, nullptr) == SGC_EINVAL);
    CHECK(sgc_encode(L, 0, 6, nullptr, Al, cap, Au, wb, Aq, Aq, Aq, cb, nullptr, A, eneed, nullptr) == SGC_EINVAL);
    CHECK(sgc_encode(L, 0, 6, Ai, Al, cap, Au, wb - 1, Aq, Aq, Aq, cb, nullptr, A, eneed, nullptr) == SGC_ENOSPC);
    CHECK(sgc_encode(L, 0, 6, Ai, Al, cap, Au, wb, Aq, Aq, Aq, 0, nullptr, A, eneed, nullptr) == SGC_ENOSPC);
    CHECK(sgc_encode(L, 0, 6, Ai, Al, cap, Au, wb, Aq, Aq, Aq, cb, nullptr, A, eneed - 1, nullptr) == SGC_ENOSPC);

    sgc_message m = {SGC_MSG_RAW_F32, 0, 0, 0, 10, Al, Ai, Af, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr};
    const size_t dneed = sgc_decode_accumulate_workspace(L, &m, 1);
    CHECK(dneed > 0);
    CHECK(sgc_decode_accumulate(L, &m, 1, 5, Af, Af, nullptr, A, dneed, nullptr) == SGC_EINVAL);
    CHECK(sgc_decode_accumulate(L, &m, 1, 0, Af, (float*)MIS, nullptr, A, dneed, nullptr) == SGC_EINVAL);
    CHECK(sgc_decode_accumulate(L, &m, 1, SGC_INIT_BASE, nullptr, Af, nullptr, A, dneed, nullptr) == SGC_EINVAL);
    CHECK(sgc_decode_accumulate(L, &m, 1, 0, Af, Af, nullptr, A, dneed - 1, nullptr) == SGC_ENOSPC);
    CHECK(sgc_decode_accumulate(L, &m, -1, 0, Af, Af, nullptr, A, dneed, nullptr) == SGC_EINVAL);
    sgc_message badf = m;
    badf.format = 9;
    CHECK(sgc_decode_accumulate(L, &badf, 1, 0, Af, Af, nullptr, A, dneed, nullptr) == SGC_EINVAL);
    CHECK(sgc_decode_accumulate_workspace(L, &badf, 1) == 0);
    sgc_message nov = m;
    nov.val = nullptr;
    CHECK(sgc_decode_accumulate(L, &nov, 1, 0, Af, Af, nullptr, A, dneed, nullptr) == SGC_EINVAL);
    sgc_message gol = {SGC_MSG_GOLOMB_F32, 0, 40, 0, 10, Al, nullptr, Af, nullptr, nullptr, Au, Aq, Aq, Aq};
    CHECK(sgc_decode_accumulate(L, &gol, 1, 0, Af, Af, nullptr, A, dneed, nullptr) == SGC_EINVAL);
    CHECK(sgc_set_pass_events(A, nullptr) == SGC_EINVAL);
    CHECK(sgc_set_pass_events(nullptr, nullptr) == SGC_OK);
    sgc_layout_destroy(L);

    if (failures) {
        std::fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    std::printf("abi driver ok\n");
    return 0;
}
