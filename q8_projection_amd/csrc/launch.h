// launch.h -- launchers of the HIP kernels, called by the validated C ABI.
// Every launcher enqueues on `stream` and returns hipGetLastError()'s result.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q8 {

// Device facts the launchers size grids with (cached per device).
struct DeviceInfo {
    int cus;             // compute units
    int lds_per_block;   // bytes of LDS one workgroup may use
};
DeviceInfo device_info();

// Bytes of the counters at the head of a K-split workspace: one u32 per 16-row
// tile of the tallest matrix that splits (16 rows per CU), so that every
// split's row ranges find their counters there, rounded up to 16 bytes.
inline int64_t split_count_bytes(int cus) { return (int64_t(cus) * 4 + 15) / 16 * 16; }

hipError_t launch_quantize_weights(const float *w, int64_t n, int64_t k, uint8_t *blocks,
                                   hipStream_t stream);
hipError_t launch_quantize_act(int words, const float *x, int64_t rows, int64_t k, int8_t *hi,
                               int8_t *lo, float *scale, hipStream_t stream);

// Projection of up to 8 rows with the int8 dot4 GEMV kernels (integer modes)
// or the f64 GEMV (f32 mode).  mode: 0 f32, 1 one-word, 2 two-word.
// With `argmax` (one row, resident stack, one launch): also write argmax_i y[i]
// (lowest i among equal maxima) there, using `argmax_work` (gemv_argmax_work_bytes,
// zero-filled before its first use and left zero-filled).
hipError_t launch_gemv(int mode, const uint8_t *w, int64_t n, int64_t k, int rows, const int8_t *hi,
                       const int8_t *lo, const float *scale, const float *x, const float *residual,
                       float *y, hipStream_t stream, int32_t *argmax = nullptr, void *argmax_work = nullptr);
// Workgroups of the one-row resident launch over n weight rows.
int64_t gemv_row_grid(int64_t n);
// Whether the one-row projection over k columns keeps its stack resident in LDS
// (a single launch that can finish with the fused arg-max).
bool gemv_row_resident(int mode, int64_t k);

// The block sums of the integer modes as the GEMV kernel that would project
// this call computes them (words 1 or 2, rows 1..8): sums [rows][sums_ld][k/32]
// [words], this launch's n weight rows starting at row 0 of the export.
hipError_t launch_gemv_sums(int words, const uint8_t *w, int64_t n, int64_t k, int rows, const int8_t *hi,
                            const int8_t *lo, int32_t *sums, int64_t sums_ld, hipStream_t stream);

// Projection of 2..64 rows with the LDS-staged int8 MFMA kernel (integer
// modes).  y and residual have row stride ldy.
hipError_t launch_mma(int mode, const uint8_t *w, int64_t n, int64_t k, int rows, const int8_t *hi,
                      const int8_t *lo, const float *scale, const float *residual, float *y, int64_t ldy,
                      hipStream_t stream);
// The block sums of the same call as the MFMA kernel that launch_mma picks
// computes them: sums [rows][n][k/32][words] (words 2 in the two-word mode).
// Needs what mma_supports needs, with hi standing in for the scales.
hipError_t launch_mma_sums(int mode, const uint8_t *w, int64_t n, int64_t k, int rows, const int8_t *hi,
                           const int8_t *lo, int32_t *sums, hipStream_t stream);
// Whether launch_mma serves this call: integer mode, 3..64 rows (and stacks of
// 2 rows on a matrix of at most 16 rows per CU, or whose row ranges fill at
// least three quarters of their MFMA tiles (two-word) or whole 64-row ranges
// (one-word); the GEMV is faster for the other 2-row stacks), k a multiple of
// 256, and weights, words and scales 16-byte aligned.  Weights of 1 GiB or more
// run as row slices of under 1 GiB, one launch each.
bool mma_supports(int mode, int64_t n, int64_t k, int rows, const void *w, const void *hi, const void *lo,
                  const void *scale);
// The same projection with K split over workgroups, for stacks of 2..64 rows
// on a matrix short enough that launch_mma gives each workgroup a single
// 16-row tile: 64-row ranges, each range's K split over 2, 4 or 8 workgroups
// whose f64 partials meet in `workspace` and are added in split order by the
// last to arrive.  mma_ksplit_bytes: the workspace this call needs, 0 where it
// does not split (then launch_mma serves it).  The workspace's counters must be
// zero before the launch; the launch leaves them zero.
int64_t mma_ksplit_bytes(int mode, int64_t n, int64_t k, int rows);
hipError_t launch_mma_ksplit(int mode, const uint8_t *w, int64_t n, int64_t k, int rows, const int8_t *hi,
                             const int8_t *lo, const float *scale, const float *residual, float *y, void *workspace,
                             hipStream_t stream);

// Projection of a stack of 5..64 f32 rows (f32 mode, f64 sums) on the f64
// MFMA kernel, every weight block read once.  y and residual have row stride
// ldy.  Needs what f64_mma_supports needs.
hipError_t launch_f64_mma(const uint8_t *w, int64_t n, int64_t k, int rows, const float *x, const float *residual,
                          float *y, int64_t ldy, hipStream_t stream);
// The f32 stack with K split over workgroups, for matrices of at most 16 rows
// per CU (where launch_f64_mma keeps one weight tile a workgroup): two tiles a
// workgroup, each range's K over 2, 4 or 8 workgroups, partials combined in
// split order in `workspace` as launch_mma_ksplit does.  f64_ksplit_bytes: the
// workspace it needs, 0 where it does not split.  y and residual have row
// stride n.
int64_t f64_ksplit_bytes(int64_t n, int64_t k, int rows);
hipError_t launch_f64_mma_ksplit(const uint8_t *w, int64_t n, int64_t k, int rows, const float *x,
                                 const float *residual, float *y, void *workspace, hipStream_t stream);
// Whether launch_f64_mma serves this stack: 5..64 rows, n >= 1, k a multiple of
// 64 up to 2^22, x 16-byte aligned.
bool f64_mma_supports(int64_t n, int64_t k, int rows, const void *x);

// The fixed device array that stands in for the fused arg-max's workspace in
// q8_matvec_argmax_noalloc: its size, its address on the current device
// (looked up once per device), and a kernel that clears its counter.
int64_t argmax_scratch_bytes();
hipError_t argmax_scratch(void **out);
hipError_t launch_clear_argmax_header(void *workspace, hipStream_t stream);


}  // namespace q8
