// gemv_i8x2.hip -- the GEMV kernels of the two-word int8 mode, rows 1..8.
#include "gemv_kernels.h"

namespace q8 {
hipError_t gemv_dispatch_i8x2(int rows, const GemvArgs &a, hipStream_t s) { return dispatch_int<2>(rows, a, s); }
}  // namespace q8
