// bf16 I/O path of the GMA forward (MFMA kernels).  Placeholder: not implemented yet.
#include "gma_internal.h"

namespace gma {
hipError_t bf16_responsibilities(const Plan&, const void*, const float*, const float*, const float*, void*,
                                 gma_dtype_t, char*, hipStream_t) { return hipErrorNotSupported; }
hipError_t bf16_bidir(const Plan&, const void*, const void*, const void*, const float*, const float*,
                      const float*, float, void*, char*, hipStream_t) { return hipErrorNotSupported; }
hipError_t bf16_causal(const Plan&, const void*, const void*, const void*, const float*, const float*,
                       const float*, float, void*, char*, hipStream_t) { return hipErrorNotSupported; }
}  // namespace gma
