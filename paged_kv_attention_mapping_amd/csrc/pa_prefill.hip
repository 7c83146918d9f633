// pa_prefill.hip -- MFMA flash-attention prefill (bf16).  Placeholder: the
// vector-ALU row path serves every shape until the MFMA kernel lands.
#include "pa_device.h"
#include "pa_kernels.h"

namespace pa {

bool prefill_mfma_supported(const PoolGeom &, int) { return false; }

hipError_t launch_prefill_mfma(const void *, int64_t, int, const void *, const void *, const PoolGeom &,
                               const int32_t *, const int32_t *, const int32_t *, const int32_t *, int,
                               int, int, int, float, void *, hipStream_t) {
    return hipErrorInvalidValue;
}

}  // namespace pa
