// Stand-ins for the library's kernel launchers, linked into the host-only
// sanitizer build of api.cpp (tests/sanitize/api_driver.cpp).  The driver
// runs without a GPU, where every entry point returns before reaching them;
// they never launch anything and report an error if reached.
#include <hip/hip_runtime.h>

#include <string>

#include "../../moe_grouped_gemm_scaled_amd/csrc/dg_internal.h"

namespace dg {

hipError_t launch_quant_1x128(const float *, int, int, int, uint8_t *, float *, int, hipStream_t, bool) {
    return hipErrorInvalidValue;
}
hipError_t launch_quant_128x128(const float *, int, int, int, uint8_t *, float *, hipStream_t, bool) {
    return hipErrorInvalidValue;
}
hipError_t launch_mqa_logits(const uint8_t *, const uint8_t *, const float *, const float *, const int32_t *,
                             const int32_t *, int, float *, int, int, int, hipStream_t, std::string &config) {
    config = "stub";
    return hipErrorInvalidValue;
}
hipError_t launch_gemm(const GemmProblem &, int, hipStream_t, std::string &config) {
    config = "stub";
    return hipErrorInvalidValue;
}
hipError_t launch_pack_ue8m0(const float *, int, int, int, uint32_t *, hipStream_t) { return hipErrorInvalidValue; }
hipError_t noalloc_scratch(hipStream_t, void **, size_t *) { return hipErrorInvalidValue; }

}  // namespace dg
