// Causal chunked scan of the bf16 path (placeholder until the MFMA scan lands).
#include "gma_internal.h"

namespace gma {
hipError_t bf16_scan(const Plan&, const void*, const void*, const void*, const uint16_t*, const float*, float, void*,
                     char*, hipStream_t) {
    return hipErrorNotSupported;
}
}  // namespace gma
