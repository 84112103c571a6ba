// sums.hip -- the exact int32 block dot products of the integer modes for the
// GEMV kernels that have no export of their own (unaligned weights, or a stack
// staged in column tiles): one thread per weight block, with those kernels'
// block decode (36-byte window load, v_perm realignment) and v_dot4 chain.
#include "device.h"
#include "launch.h"

namespace q8 {
namespace {

constexpr int kThreads = 256;

template <int WORDS>
__global__ __launch_bounds__(kThreads) void block_sums_kernel(const uint8_t *__restrict__ w, int64_t n,
                                                              int k, int64_t rows,
                                                              const int8_t *__restrict__ hi,
                                                              const int8_t *__restrict__ lo,
                                                              int32_t *__restrict__ sums, int64_t ld) {
    const int nb = k / kBlock;
    const int64_t g = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    if (g >= n * nb) return;
    const int64_t row = g / nb;
    const int b = static_cast<int>(g % nb);
    Window win;
    load_window(w, g, win);
    uint32_t q[8];
    window_quants(win, window_selector(g), q);
    for (int64_t r = 0; r < rows; ++r) {
        uint32_t a[8];
        const uint32_t *ph = reinterpret_cast<const uint32_t *>(hi + r * k + b * kBlock);
#pragma unroll
        for (int j = 0; j < 8; ++j) a[j] = ph[j];
        int32_t *out = sums + ((r * ld + row) * nb + b) * WORDS;
        out[0] = dot32(q, a);
        if (WORDS == 2) {
            const uint32_t *pl = reinterpret_cast<const uint32_t *>(lo + r * k + b * kBlock);
#pragma unroll
            for (int j = 0; j < 8; ++j) a[j] = pl[j];
            out[1] = dot32(q, a);
        }
    }
}

}  // namespace

hipError_t launch_block_sums(int words, const uint8_t *w, int64_t n, int64_t k, int64_t rows,
                             const int8_t *hi, const int8_t *lo, int32_t *sums, int64_t sums_ld,
                             hipStream_t stream) {
    const int64_t total = n * (k / kBlock);
    const dim3 grid(static_cast<unsigned>((total + kThreads - 1) / kThreads));
    if (words == 2)
        block_sums_kernel<2><<<grid, kThreads, 0, stream>>>(w, n, static_cast<int>(k), rows, hi, lo, sums, sums_ld);
    else
        block_sums_kernel<1><<<grid, kThreads, 0, stream>>>(w, n, static_cast<int>(k), rows, hi, lo, sums, sums_ld);
    return hipGetLastError();
}

}  // namespace q8
