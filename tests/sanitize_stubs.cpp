// Launchers that launch nothing, for the sanitizer build of the library's
// argument checks (tests/test_sanitizers.py): every call that passes the
// checks and finds a gfx950 ends here with an error status instead of a
// kernel.
#include <hip/hip_runtime.h>

#include "kernels.hpp"

namespace gg {

hipError_t launch_gemm(bool, bool, int, int, int, float, const float *, int64_t, const float *,
                       int64_t, float, float *, int64_t, int, hipStream_t) {
    return hipErrorNotSupported;
}

hipError_t launch_gemv_f32(int, int, int, const float *const *, int64_t, const float *const *,
                           float *const *, hipStream_t) {
    return hipErrorNotSupported;
}

hipError_t launch_gemv_q2(int, int, int, const uint8_t *const *, int64_t, const uint16_t *const *,
                          int64_t, const float *const *, float *const *, float *, hipStream_t) {
    return hipErrorNotSupported;
}

hipError_t launch_gemv_q4(int, int, int, const uint8_t *const *, int64_t, const uint16_t *const *,
                          int64_t, const float *const *, float *const *, hipStream_t) {
    return hipErrorNotSupported;
}

float *device_scratch() { return nullptr; }

}  // namespace gg
