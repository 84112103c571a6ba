// gemv_i8.hip -- the GEMV kernels of the one-word int8 mode, rows 1..8.
#include "gemv_kernels.h"

namespace q8 {
hipError_t gemv_dispatch_i8(int rows, const GemvArgs &a, hipStream_t s) { return dispatch_int<1>(rows, a, s); }
}  // namespace q8
