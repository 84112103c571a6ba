// gemv.hip -- launchers of the GEMV family (stacks of 1..8 activation rows):
// argument packing and the dispatch by activation mode.  The kernels are in
// gemv_kernels.h; gemv_f32.hip, gemv_i8.hip, gemv_i8x2.hip and gemv_sums.hip
// instantiate them.
#include "gemv_kernels.h"

namespace q8 {

bool gemv_row_resident(int mode, int64_t k) {
    const int words = mode == 0 ? 0 : mode;
    return tile_columns(static_cast<int>(k), 1, words) >= k;
}

int64_t gemv_row_grid(int64_t n) {
    // as run<1, WORDS, 1, P> sizes the resident grid: one group per row
    const int64_t waves = std::max<int64_t>(std::min<int64_t>(n, static_cast<int64_t>(device_info().cus) * kWavesPerCu),
                                            (n + kOutPerWave - 1) / kOutPerWave);
    return (waves + kWaves - 1) / kWaves;
}

hipError_t launch_gemv(int mode, const uint8_t *w, int64_t n, int64_t k, int rows, const int8_t *hi,
                       const int8_t *lo, const float *scale, const float *x, const float *residual,
                       float *y, hipStream_t stream, int32_t *argmax, void *argmax_work) {
    GemvArgs a{};
    a.argmax = argmax;
    a.argmax_work = static_cast<uint32_t *>(argmax_work);
    a.w = w;
    a.hi = hi;
    a.lo = lo;
    a.scale = scale;
    a.x = x;
    a.residual = residual;
    a.y = y;
    a.n = n;
    a.ldy = n;
    a.k = static_cast<int>(k);
    a.nb = static_cast<int>(k / kBlock);
    if (mode == 0) return gemv_dispatch_f32(rows, a, stream);
    if (mode == 2) return gemv_dispatch_i8x2(rows, a, stream);
    return gemv_dispatch_i8(rows, a, stream);
}

hipError_t launch_gemv_sums(int words, const uint8_t *w, int64_t n, int64_t k, int rows, const int8_t *hi,
                            const int8_t *lo, int32_t *sums, int64_t sums_ld, hipStream_t stream) {
    GemvArgs a{};
    a.w = w;
    a.hi = hi;
    a.lo = lo;
    a.n = n;
    a.ldy = n;
    a.k = static_cast<int>(k);
    a.nb = static_cast<int>(k / kBlock);
    a.sums = sums;
    a.sums_ld = sums_ld;
    return gemv_dispatch_sums(words, rows, a, stream);
}

}  // namespace q8
