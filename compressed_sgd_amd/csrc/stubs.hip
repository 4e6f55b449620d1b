// stubs.hip -- entry points not built yet (return SGC_EUNSUPPORTED).
#include "sgc_common.h"
extern "C" size_t sgc_binarize_workspace(const sgc_layout*, int64_t) { return 0; }
extern "C" int sgc_binarize(const sgc_layout*, int32_t, const int32_t*, const float*, const int64_t*, int64_t, float*,
                            int32_t*, int64_t*, float*, uint32_t*, void*, size_t, sgc_stream_t) { return SGC_EUNSUPPORTED; }
extern "C" int64_t sgc_encode_word_bound(const sgc_layout*, int32_t, int32_t, int64_t) { return -1; }
extern "C" int64_t sgc_encode_chunk_bound(const sgc_layout*, int32_t, int64_t) { return -1; }
extern "C" size_t sgc_encode_workspace(const sgc_layout*, int32_t, int64_t) { return 0; }
extern "C" int sgc_encode(const sgc_layout*, int32_t, int32_t, const int32_t*, const int64_t*, int64_t, uint32_t*, int64_t,
                          uint64_t*, uint64_t*, uint64_t*, int64_t, uint32_t*, void*, size_t, sgc_stream_t) { return SGC_EUNSUPPORTED; }
extern "C" size_t sgc_decode_accumulate_workspace(const sgc_layout*, const sgc_message*, int32_t) { return 0; }
extern "C" int sgc_decode_accumulate(const sgc_layout*, const sgc_message*, int32_t, int32_t, const float*, float*,
                                     uint32_t*, void*, size_t, sgc_stream_t) { return SGC_EUNSUPPORTED; }
