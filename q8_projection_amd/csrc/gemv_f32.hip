// gemv_f32.hip -- the GEMV kernels of the f32 mode (f64 sums), rows 1..8.
#include "gemv_kernels.h"

namespace q8 {

hipError_t gemv_dispatch_f32(int rows, const GemvArgs &a, hipStream_t s) {
    // one weight row a wave group (MR 1), items in flight per stack height
    switch (rows) {
        case 1: return run<1, 0, 1, 2>(a, s);
        case 2: return run<2, 0, 1, 4>(a, s);
        case 3: return run<3, 0, 1, 4>(a, s);
        case 4: return run<4, 0, 1, 4>(a, s);
        case 5: return run<5, 0, 1, 2>(a, s);
        case 6: return run<6, 0, 1, 2>(a, s);
        case 7: return run<7, 0, 1, 2>(a, s);
        default: return run<8, 0, 1, 2>(a, s);
    }
}

}  // namespace q8
