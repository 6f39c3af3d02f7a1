// Causal varlen prefill over the paged cache (placeholder until the MFMA kernel).
#include "pa_launch.h"

namespace pa {

hipError_t launch_prefill(const uint16_t*, const uint8_t*, const uint8_t*, const int32_t*,
                          const int32_t*, const int32_t*, int, int, int, int, int, float,
                          uint16_t*, const PoolDims&, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace pa
