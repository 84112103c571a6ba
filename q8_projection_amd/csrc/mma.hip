// mma.hip -- launchers of the int8 MFMA projection (stacks of 2..64 rows);
// the kernels are in mma_kernels.h.
#include "mma_kernels.h"

namespace q8 {

bool mma_supports(int mode, int64_t n, int64_t k, int rows, const void *w, const void *hi, const void *lo,
                  const void *scale) {
    if (mode != 1 && mode != 2) return false;
    if (rows < 2 || rows > 64 || k % (kChunkBlocks * kBlock) != 0) return false;
    // Measured crossover with the GEMV at two rows: the MFMA kernels are faster
    // on a matrix short enough that a workgroup owns a single 16-row tile (the
    // wave-private kernel), and on taller ones where the workgroups fill at least
    // three quarters of their 32- or 64-row tile range (two-word) or all 64 rows
    // (one-word); elsewhere the GEMV is.
    const int64_t cus = std::max(1, device_info().cus);
    const int64_t per_wg = std::min<int64_t>((n + cus - 1) / cus, 64);
    const int64_t tile_rows = per_wg <= 16 ? 16 : per_wg <= 32 ? 32 : 64;
    const bool one_tile = per_wg <= 16;
    const bool two_rows = one_tile || (mode == 2 ? 4 * per_wg >= 3 * tile_rows : per_wg == 64);
    if (rows == 2 && !two_rows) return false;
    // launches take row slices under 1 GiB of weights; a 16-row slice must fit
    if (16 * (k / kBlock) * kBlockBytes > (int64_t(1) << 30)) return false;
    const auto al16 = [](const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
    if (!al16(w) || !al16(hi) || !al16(scale) || (mode == 2 && !al16(lo))) return false;
    return true;
}

hipError_t launch_mma(int mode, const uint8_t *w, int64_t n, int64_t k, int rows, const int8_t *hi,
                      const int8_t *lo, const float *scale, const float *residual, float *y, int64_t ldy,
                      hipStream_t stream) {
    return launch_mma_impl<false>(mode, w, n, k, rows, hi, lo, scale, residual, y, ldy, nullptr, stream);
}

int64_t mma_ksplit_bytes(int mode, int64_t n, int64_t k, int rows) {
    if (rows < 2) return 0;
    const KsPlan p = ks_plan(mode, n, k, rows);
    return p.ksplit > 1 ? p.bytes : 0;
}

hipError_t launch_mma_ksplit(int mode, const uint8_t *w, int64_t n, int64_t k, int rows, const int8_t *hi,
                             const int8_t *lo, const float *scale, const float *residual, float *y, void *workspace,
                             hipStream_t stream) {
    return launch_mma_ksplit_impl(mode, w, n, k, rows, hi, lo, scale, residual, y, n, workspace, stream);
}

}  // namespace q8
