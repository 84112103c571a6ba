// mma_sums.hip -- the block-sum export of the int8 MFMA kernels: the kernel and
// wave split that project a call write its exact int32 block sums.
#include "mma_kernels.h"

namespace q8 {

hipError_t launch_mma_sums(int mode, const uint8_t *w, int64_t n, int64_t k, int rows, const int8_t *hi,
                           const int8_t *lo, int32_t *sums, hipStream_t stream) {
    return launch_mma_impl<true>(mode, w, n, k, rows, hi, lo, nullptr, nullptr, nullptr, n, sums, stream);
}

}  // namespace q8
