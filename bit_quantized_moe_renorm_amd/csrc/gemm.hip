// gemm.hip - prefill path: grouped dequant MFMA GEMMs (not yet enabled).
#include "common.h"

namespace ds4 {

bool gemm_enabled() { return false; }

hipError_t launch_gemm_gateup(const Layer &, const Work &, const void *, int, hipStream_t) {
    return hipErrorNotSupported;
}
hipError_t launch_gemm_down(const Layer &, const Work &, int, float *, hipStream_t) {
    return hipErrorNotSupported;
}

}  // namespace ds4
