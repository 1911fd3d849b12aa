// L = 16 register-resident Viterbi path (placeholder until the kernel lands).
#include <hip/hip_runtime.h>

#include "tcq.h"
#include "tcq_internal.h"

namespace tcq {

bool l16_supported(const Problem &) { return false; }
size_t l16_fixed_bytes(const Problem &) { return 0; }
size_t l16_bp_bytes(const Problem &) { return 0; }
hipError_t launch_l16_prepare(const Problem &, const float *, char *, hipStream_t) {
    return hipErrorNotSupported;
}
hipError_t launch_acs_l16(const Problem &, const Plan &, const float *, const float *, int64_t,
                          int64_t, char *, float *, hipStream_t) {
    return hipErrorNotSupported;
}
hipError_t launch_traceback_l16(const Problem &, const Plan &, int64_t, int64_t, const char *,
                                uint32_t *, uint32_t *, hipStream_t) {
    return hipErrorNotSupported;
}

}  // namespace tcq
