// gemv_sums.hip -- the block-sum export of the GEMV kernels (integer modes,
// rows 1..8): the kernel that projects a call writes its int32 block sums.
#include "gemv_kernels.h"

namespace q8 {
hipError_t gemv_dispatch_sums(int words, int rows, const GemvArgs &a, hipStream_t s) {
    return words == 2 ? dispatch_int<2, true>(rows, a, s) : dispatch_int<1, true>(rows, a, s);
}
}  // namespace q8
