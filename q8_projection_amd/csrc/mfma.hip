// mfma.hip -- the projection for wide stacks (prefill chunks) on int8 MFMA.
#include "device.h"
#include "launch.h"

namespace q8 {

bool mfma_supports(int, int) { return false; }

hipError_t launch_mfma(int, const uint8_t *, int64_t, int64_t, int, const int8_t *, const int8_t *,
                       const float *, const float *, float *, hipStream_t) {
    return hipErrorNotSupported;
}

}  // namespace q8
