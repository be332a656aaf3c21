// Launch functions for the AddressSanitizer build of the host library
// (tests/test_asan_host.py): the C ABI's host checks and plans are linked
// as they are, and every launch aborts, since the checks under test must
// return before any launch.
#include <stdlib.h>

#include "kernels.hpp"

namespace attn {

hipError_t launch_decode(const DecodePlan &, const float *, const float *, const float *,
                         float *, uint32_t, uint32_t, uint32_t, uint32_t, uint32_t, float,
                         void *, const DecodeAppend *, hipStream_t, const DecodeVarlen *) {
    abort();
}

hipError_t launch_prefill(const PrefillPlan &, const float *, const float *, const float *,
                          float *, uint32_t, uint32_t, uint32_t, uint32_t, uint32_t, uint32_t,
                          hipStream_t) {
    abort();
}

hipError_t launch_kv_append(const float *, const float *, float *, float *, uint32_t, uint32_t,
                            uint32_t, uint32_t, uint32_t, hipStream_t, const float *,
                            const float *, const uint32_t *, uint32_t) {
    abort();
}

hipError_t launch_kv_append_rows(const float *, const float *, float *, float *, uint32_t,
                                 uint32_t, uint32_t, uint32_t, uint32_t, uint32_t,
                                 hipStream_t) {
    abort();
}

}  // namespace attn
