// abi.cpp -- the C ABI of libq8proj.so: argument validation, then dispatch to
// the HIP launchers on the caller's stream.  Nothing here allocates, frees,
// synchronizes or reads device memory (codegen_cuda::lane page, Modules: arena;
// every call can be captured into a graph, as the lane captures each step).
// Errors are named (codegen_cuda::lane page, Enums: LaneError) and returned
// before anything is enqueued.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>

#include "../../include/q8.h"
#include "launch.h"

namespace {

constexpr int64_t kMaxK = int64_t(1) << 24;           // columns
constexpr int64_t kMaxBlocks = int64_t(1) << 27;      // n * k/32 (4.5 GB of weights)
constexpr int64_t kMaxRowsTimesN = int64_t(1) << 31;  // elements of y
constexpr int64_t kMaxInsideRows = 8;                 // integer stacks quantized inside a projection
constexpr int kMaxDevices = 64;

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Do byte ranges [a, a+an) and [b, b+bn) overlap?
bool overlap(const void *a, int64_t an, const void *b, int64_t bn) {
    if (!a || !b || an <= 0 || bn <= 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + static_cast<uintptr_t>(bn) && b0 < a0 + static_cast<uintptr_t>(an);
}

q8_status check_k(int64_t k) {
    if (k <= 0 || k % 64 != 0 || k > kMaxK) return Q8_E_SHAPE;
    return Q8_OK;
}

// Sizes of a projection, each bounded before any product of them is formed:
// n * k/32 <= kMaxBlocks, rows * n <= kMaxRowsTimesN and rows <= 2^25, so
// every byte count below fits int64 with room to spare.
q8_status check_sizes(int64_t n, int64_t k, int64_t rows) {
    if (n < 0 || rows < 0) return Q8_E_SHAPE;
    if (q8_status s = check_k(k); s != Q8_OK) return s;
    if (n > kMaxBlocks / (k / 32)) return Q8_E_SHAPE;
    if (rows > kMaxRowsTimesN / 64) return Q8_E_SHAPE;
    if (n > 0 && rows > kMaxRowsTimesN / n) return Q8_E_SHAPE;
    return Q8_OK;
}

q8_status from_hip(hipError_t e) { return e == hipSuccess ? Q8_OK : Q8_E_HIP; }

hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }

// Validation shared by q8_matvec / q8_matmul_rows / q8_block_sums.
q8_status check_projection(int mode, const void *w, int64_t n, int64_t k, int64_t rows, const int8_t *hi,
                           const int8_t *lo, const float *scale, const float *x, const float *residual,
                           const void *out, int64_t out_bytes, bool f32_allowed, bool need_scale) {
    if (mode != Q8_ACT_F32 && mode != Q8_ACT_I8 && mode != Q8_ACT_I8X2) return Q8_E_MODE;
    if (mode == Q8_ACT_F32 && !f32_allowed) return Q8_E_MODE;
    if (q8_status s = check_sizes(n, k, rows); s != Q8_OK) return s;
    const int64_t nb = k / 32;
    if (!w || !out) return Q8_E_NULL;
    // Integer modes take the quantized stack (hi, lo, scale) or, with all three
    // null, the f32 stack x to quantize inside the projection.
    const bool quantize_inside = mode != Q8_ACT_F32 && f32_allowed && !hi && !lo && !scale && x;
    if (mode == Q8_ACT_F32 || quantize_inside) {
        if (!x) return Q8_E_NULL;
    } else {
        if (!hi || (need_scale && !scale)) return Q8_E_NULL;
        if (mode == Q8_ACT_I8X2 && !lo) return Q8_E_NULL;
    }
    if (!aligned(w, 4) || !aligned(out, 4)) return Q8_E_ALIGN;
    if (residual && !aligned(residual, 4)) return Q8_E_ALIGN;
    if (mode == Q8_ACT_F32 || quantize_inside) {
        if (!aligned(x, 16)) return Q8_E_ALIGN;
    } else {
        if (!aligned(hi, 16) || (need_scale && !aligned(scale, 4))) return Q8_E_ALIGN;
        if (mode == Q8_ACT_I8X2 && !aligned(lo, 16)) return Q8_E_ALIGN;
    }
    const int64_t wbytes = n * nb * 34;
    const int64_t abytes = rows * k;
    if (overlap(out, out_bytes, w, wbytes)) return Q8_E_ALIAS;
    if (mode == Q8_ACT_F32 || quantize_inside) {
        if (overlap(out, out_bytes, x, abytes * 4)) return Q8_E_ALIAS;
    } else {
        if (overlap(out, out_bytes, hi, abytes)) return Q8_E_ALIAS;
        if (need_scale && overlap(out, out_bytes, scale, rows * nb * 4)) return Q8_E_ALIAS;
        if (mode == Q8_ACT_I8X2 && overlap(out, out_bytes, lo, abytes)) return Q8_E_ALIAS;
    }
    if (residual && residual != out && overlap(out, out_bytes, residual, rows * n * 4)) return Q8_E_ALIAS;
    return Q8_OK;
}

// Which kernel family projects a slice of at most 64 rows.  The projection and
// the block-sum export both ask here, so the export runs the projection's
// kernels.
bool mma_serves(int mode, int64_t n, int64_t k, int rows, const void *w, const int8_t *hi, const int8_t *lo,
                const void *scale, bool quantize_inside) {
    return !quantize_inside && q8::mma_supports(mode, n, k, rows, w, hi, lo, scale);
}

// One slice of at most 64 rows of q8_matmul_rows (pointers at the slice's first
// row): the int8 MFMA kernels, the f64 MFMA kernel, or the GEMV family 8 rows at
// a time.
hipError_t project_slice(int mode, const uint8_t *wb, int64_t n, int64_t k, int r, const int8_t *shi,
                         const int8_t *slo, const float *ssc, const float *sx, const float *sres, float *sy,
                         bool inside, hipStream_t st) {
    if (mma_serves(mode, n, k, r, wb, shi, slo, ssc, inside))
        return q8::launch_mma(mode, wb, n, k, r, shi, slo, ssc, sres, sy, n, st);
    if (mode == Q8_ACT_F32 && q8::f64_mma_supports(n, k, r, sx))
        return q8::launch_f64_mma(wb, n, k, r, sx, sres, sy, n, st);
    const int64_t nb = k / 32;
    hipError_t e = hipSuccess;
    for (int c0 = 0; c0 < r && e == hipSuccess; c0 += 8) {
        const int c = std::min(8, r - c0);
        e = q8::launch_gemv(mode, wb, n, k, c, shi ? shi + c0 * k : nullptr, slo ? slo + c0 * k : nullptr,
                            ssc ? ssc + c0 * nb : nullptr, sx ? sx + c0 * k : nullptr,
                            sres ? sres + c0 * n : nullptr, sy + c0 * n, st);
    }
    return e;
}

}  // namespace

namespace q8 {

// Per-device attributes, queried once.  The cache entry packs both values in
// one atomic word, so concurrent first calls from several host threads each
// store the same value and no caller sees one field without the other.
DeviceInfo device_info() {
    static std::atomic<uint64_t> cache[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) dev = 0;
    uint64_t v = cache[dev].load(std::memory_order_acquire);
    if (v == 0) {
        int cus = 0, lds = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = 256;
        if (hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess || lds <= 0)
            lds = 64 * 1024;
        v = (static_cast<uint64_t>(static_cast<uint32_t>(lds)) << 32) | static_cast<uint32_t>(cus);
        cache[dev].store(v, std::memory_order_release);
    }
    DeviceInfo d;
    d.cus = static_cast<int>(static_cast<uint32_t>(v));
    d.lds_per_block = static_cast<int>(v >> 32);
    return d;
}

}  // namespace q8

extern "C" {

q8_status q8_quantize_weights(const float *w, int64_t n, int64_t k, void *blocks, void *stream) {
    if (n < 0) return Q8_E_SHAPE;
    if (q8_status s = check_k(k); s != Q8_OK) return s;
    if (n > kMaxBlocks / (k / 32)) return Q8_E_SHAPE;
    if (!w || !blocks) return Q8_E_NULL;
    if (!aligned(w, 4) || !aligned(blocks, 4)) return Q8_E_ALIGN;
    if (overlap(blocks, n * (k / 32) * 34, w, n * k * 4)) return Q8_E_ALIAS;
    if (n == 0) return Q8_OK;
    return from_hip(q8::launch_quantize_weights(w, n, k, static_cast<uint8_t *>(blocks), as_stream(stream)));
}

q8_status q8_quantize_act(int mode, const float *x, int64_t rows, int64_t k, int8_t *hi, int8_t *lo,
                          float *scale, void *stream) {
    if (mode != Q8_ACT_I8 && mode != Q8_ACT_I8X2) return Q8_E_MODE;
    if (rows < 0) return Q8_E_SHAPE;
    if (q8_status s = check_k(k); s != Q8_OK) return s;
    if (rows > kMaxBlocks / (k / 32)) return Q8_E_SHAPE;
    if (!x || !hi || !scale || (mode == Q8_ACT_I8X2 && !lo)) return Q8_E_NULL;
    if (!aligned(x, 16) || !aligned(hi, 16) || !aligned(scale, 4) || (mode == Q8_ACT_I8X2 && !aligned(lo, 16)))
        return Q8_E_ALIGN;
    const int64_t nv = rows * k, nbk = rows * (k / 32);
    if (overlap(hi, nv, x, nv * 4) || overlap(scale, nbk * 4, x, nv * 4) || overlap(hi, nv, scale, nbk * 4))
        return Q8_E_ALIAS;
    if (mode == Q8_ACT_I8X2 &&
        (overlap(lo, nv, x, nv * 4) || overlap(lo, nv, hi, nv) || overlap(lo, nv, scale, nbk * 4)))
        return Q8_E_ALIAS;
    if (rows == 0) return Q8_OK;
    return from_hip(q8::launch_quantize_act(mode == Q8_ACT_I8X2 ? 2 : 1, x, rows, k, hi,
                                            mode == Q8_ACT_I8X2 ? lo : nullptr, scale, as_stream(stream)));
}

q8_status q8_matmul_rows(int mode, const void *w, int64_t n, int64_t k, int64_t rows, const int8_t *hi,
                         const int8_t *lo, const float *scale, const float *x, const float *residual,
                         float *y, void *stream) {
    if (q8_status s = check_sizes(n, k, rows); s != Q8_OK) return s;  // before rows * n is formed
    if (q8_status s = check_projection(mode, w, n, k, rows, hi, lo, scale, x, residual, y, rows * n * 4, true, true);
        s != Q8_OK)
        return s;
    // An integer-mode stack given as x is quantized inside the GEMV, which
    // takes at most 8 rows in one pass over the weights.
    if (mode != Q8_ACT_F32 && !hi && rows > kMaxInsideRows) return Q8_E_SHAPE;
    if (n == 0 || rows == 0) return Q8_OK;
    const uint8_t *wb = static_cast<const uint8_t *>(w);
    const int64_t nb = k / 32;
    const hipStream_t st = as_stream(stream);
    // 64-row slices, each reading every weight block once.
    for (int64_t r0 = 0; r0 < rows; r0 += 64) {
        const int r = static_cast<int>(std::min<int64_t>(64, rows - r0));
        const bool inside = mode != Q8_ACT_F32 && !hi;  // validated: x given, quantized in the kernel
        const int8_t *shi = (mode == Q8_ACT_F32 || inside) ? nullptr : hi + r0 * k;
        const int8_t *slo = (mode == Q8_ACT_I8X2 && !inside) ? lo + r0 * k : nullptr;
        const float *ssc = (mode == Q8_ACT_F32 || inside) ? nullptr : scale + r0 * nb;
        const float *sx = (mode == Q8_ACT_F32 || inside) ? x + r0 * k : nullptr;
        const float *sres = residual ? residual + r0 * n : nullptr;
        float *sy = y + r0 * n;
        if (project_slice(mode, wb, n, k, r, shi, slo, ssc, sx, sres, sy, inside, st) != hipSuccess) return Q8_E_HIP;
    }
    return Q8_OK;
}

q8_status q8_matvec(int mode, const void *w, int64_t n, int64_t k, const int8_t *hi, const int8_t *lo,
                    const float *scale, const float *x, const float *residual, float *y, void *stream) {
    return q8_matmul_rows(mode, w, n, k, 1, hi, lo, scale, x, residual, y, stream);
}

int64_t q8_matmul_rows_workspace_bytes(int mode, int64_t n, int64_t k, int64_t rows) {
    if (mode != Q8_ACT_F32 && mode != Q8_ACT_I8 && mode != Q8_ACT_I8X2) return 0;
    if (check_sizes(n, k, rows) != Q8_OK || n < 1 || rows < 2) return 0;
    // 64-row slices, one after another on the stream: the widest slice's size
    const auto bytes = [&](int r) {
        return mode == Q8_ACT_F32 ? q8::f64_ksplit_bytes(n, k, r) : q8::mma_ksplit_bytes(mode, n, k, r);
    };
    const int64_t full = bytes(static_cast<int>(std::min<int64_t>(rows, 64)));
    const int64_t tail = rows > 64 && rows % 64 ? bytes(static_cast<int>(rows % 64)) : 0;
    return std::max(full, tail);
}

q8_status q8_matmul_rows_ws(int mode, const void *w, int64_t n, int64_t k, int64_t rows, const int8_t *hi,
                            const int8_t *lo, const float *scale, const float *x, const float *residual, float *y,
                            void *workspace, int64_t workspace_bytes, void *stream) {
    if (q8_status s = check_sizes(n, k, rows); s != Q8_OK) return s;  // before rows * n is formed
    if (q8_status s = check_projection(mode, w, n, k, rows, hi, lo, scale, x, residual, y, rows * n * 4, true, true);
        s != Q8_OK)
        return s;
    const int64_t need = q8_matmul_rows_workspace_bytes(mode, n, k, rows);
    const bool inside = mode != Q8_ACT_F32 && !hi;
    // stacks this call does not split: q8_matmul_rows, the workspace untouched
    if (need == 0 || inside)
        return q8_matmul_rows(mode, w, n, k, rows, hi, lo, scale, x, residual, y, stream);
    if (!workspace) return Q8_E_NULL;
    if (!aligned(workspace, 16)) return Q8_E_ALIGN;
    if (workspace_bytes < need) return Q8_E_SHAPE;
    const int64_t nb = k / 32;
    const bool f32 = mode == Q8_ACT_F32;
    const void *ins[] = {w, f32 ? nullptr : hi, f32 ? nullptr : lo, f32 ? nullptr : scale, f32 ? x : nullptr,
                         residual, y};
    const int64_t in_bytes[] = {n * nb * 34, rows * k, mode == Q8_ACT_I8X2 ? rows * k : 0, rows * nb * 4,
                                rows * k * 4, residual ? rows * n * 4 : 0, rows * n * 4};
    for (int i = 0; i < 7; ++i)
        if (ins[i] && in_bytes[i] > 0 && overlap(workspace, need, ins[i], in_bytes[i])) return Q8_E_ALIAS;
    const uint8_t *wb = static_cast<const uint8_t *>(w);
    const hipStream_t st = as_stream(stream);
    // 64-row slices as in q8_matmul_rows; a slice that splits K uses the
    // workspace (whose counters the previous slice has returned to zero)
    for (int64_t r0 = 0; r0 < rows; r0 += 64) {
        const int r = static_cast<int>(std::min<int64_t>(64, rows - r0));
        const int8_t *shi = f32 ? nullptr : hi + r0 * k;
        const int8_t *slo = mode == Q8_ACT_I8X2 ? lo + r0 * k : nullptr;
        const float *ssc = f32 ? nullptr : scale + r0 * nb;
        const float *sx = f32 ? x + r0 * k : nullptr;
        const float *sres = residual ? residual + r0 * n : nullptr;
        float *sy = y + r0 * n;
        hipError_t e;
        if (f32 && q8::f64_ksplit_bytes(n, k, r) > 0 && q8::f64_mma_supports(n, k, r, sx))
            e = q8::launch_f64_mma_ksplit(wb, n, k, r, sx, sres, sy, workspace, st);
        else if (!f32 && q8::mma_ksplit_bytes(mode, n, k, r) > 0 && mma_serves(mode, n, k, r, wb, shi, slo, ssc, false))
            e = q8::launch_mma_ksplit(mode, wb, n, k, r, shi, slo, ssc, sres, sy, workspace, st);
        else
            e = project_slice(mode, wb, n, k, r, shi, slo, ssc, sx, sres, sy, false, st);
        if (e != hipSuccess) return Q8_E_HIP;
    }
    return Q8_OK;
}

int64_t q8_argmax_workspace_bytes(int64_t n) {
    if (n < 1 || n > INT32_MAX) return 0;
    return 16 + 8 * q8::gemv_row_grid(n);
}

}  // extern "C"

namespace {

// Validation and launch shared by the two fused arg-max entry points.  The
// workspace is the caller's (checked for alignment and overlap) or the
// library's own array (owned = false: it overlaps nothing of the caller's).
q8_status argmax_projection(int mode, const void *w, int64_t n, int64_t k, const int8_t *hi, const int8_t *lo,
                            const float *scale, const float *x, const float *residual, float *y, int32_t *idx,
                            void *workspace, bool caller_workspace, void *stream) {
    if (q8_status s = check_sizes(n, k, 1); s != Q8_OK) return s;  // before n * 4 is formed
    if (q8_status s = check_projection(mode, w, n, k, 1, hi, lo, scale, x, residual, y, n * 4, true, true);
        s != Q8_OK)
        return s;
    if (n < 1 || n > INT32_MAX) return Q8_E_SHAPE;
    // one launch: the weights in one buffer and the stack resident in LDS
    if (n * (k / 32) * 34 > (int64_t(1) << 30) || !q8::gemv_row_resident(mode, k)) return Q8_E_SHAPE;
    if (!idx || (caller_workspace && !workspace)) return Q8_E_NULL;
    if (!aligned(idx, 4) || (caller_workspace && !aligned(workspace, 16))) return Q8_E_ALIGN;
    const int64_t wsb = caller_workspace ? q8_argmax_workspace_bytes(n) : 0;
    const int64_t wbytes = n * (k / 32) * 34;
    const bool inside = mode != Q8_ACT_F32 && !hi;
    const void *ins[] = {w, hi, lo, scale, x, residual, y};
    const int64_t in_bytes[] = {wbytes, (mode == Q8_ACT_F32 || inside) ? 0 : k, (mode == Q8_ACT_I8X2 && !inside) ? k : 0,
                                (mode == Q8_ACT_F32 || inside) ? 0 : (k / 32) * 4, (mode == Q8_ACT_F32 || inside) ? k * 4 : 0,
                                residual ? n * 4 : 0, n * 4};
    for (int i = 0; i < 7; ++i)
        if (ins[i] && in_bytes[i] > 0 && (overlap(idx, 4, ins[i], in_bytes[i]) || overlap(workspace, wsb, ins[i], in_bytes[i])))
            return Q8_E_ALIAS;
    if (overlap(idx, 4, workspace, wsb)) return Q8_E_ALIAS;
    if (!caller_workspace) {
        // the library's array: at most its size, found once per device, its
        // counter cleared on this stream before the projection
        if (q8_argmax_workspace_bytes(n) > q8::argmax_scratch_bytes()) return Q8_E_SHAPE;
        if (q8::argmax_scratch(&workspace) != hipSuccess) return Q8_E_HIP;
        if (q8::launch_clear_argmax_header(workspace, as_stream(stream)) != hipSuccess) return Q8_E_HIP;
    }
    const hipError_t e = q8::launch_gemv(mode, static_cast<const uint8_t *>(w), n, k, 1,
                                         (mode == Q8_ACT_F32 || inside) ? nullptr : hi,
                                         (mode == Q8_ACT_I8X2 && !inside) ? lo : nullptr,
                                         (mode == Q8_ACT_F32 || inside) ? nullptr : scale,
                                         (mode == Q8_ACT_F32 || inside) ? x : nullptr, residual, y, as_stream(stream),
                                         idx, workspace);
    return from_hip(e);
}

}  // namespace

extern "C" {

q8_status q8_matvec_argmax(int mode, const void *w, int64_t n, int64_t k, const int8_t *hi, const int8_t *lo,
                           const float *scale, const float *x, const float *residual, float *y, int32_t *idx,
                           void *workspace, void *stream) {
    return argmax_projection(mode, w, n, k, hi, lo, scale, x, residual, y, idx, workspace, true, stream);
}

q8_status q8_matvec_argmax_noalloc(int mode, const void *w, int64_t n, int64_t k, const int8_t *hi,
                                   const int8_t *lo, const float *scale, const float *x, const float *residual,
                                   float *y, int32_t *idx, void *stream) {
    return argmax_projection(mode, w, n, k, hi, lo, scale, x, residual, y, idx, nullptr, false, stream);
}

q8_status q8_block_sums(int mode, const void *w, int64_t n, int64_t k, int64_t rows, const int8_t *hi,
                        const int8_t *lo, int32_t *sums, void *stream) {
    if (mode != Q8_ACT_I8 && mode != Q8_ACT_I8X2) return Q8_E_MODE;
    if (q8_status s = check_sizes(n, k, rows); s != Q8_OK) return s;
    const int words = mode == Q8_ACT_I8X2 ? 2 : 1;
    const int64_t nb = k / 32;
    const int64_t out_bytes = rows * n * nb * words * 4;
    if (q8_status s = check_projection(mode, w, n, k, rows, hi, lo, nullptr, nullptr, nullptr, sums, out_bytes,
                                       false, false);
        s != Q8_OK)
        return s;
    if (n == 0 || rows == 0) return Q8_OK;
    const uint8_t *wb = static_cast<const uint8_t *>(w);
    const hipStream_t st = as_stream(stream);
    // the slices and kernels q8_matmul_rows would run on this stack (the
    // scales, which the export does not take, counted as 16-byte aligned)
    for (int64_t r0 = 0; r0 < rows; r0 += 64) {
        const int r = static_cast<int>(std::min<int64_t>(64, rows - r0));
        const int8_t *shi = hi + r0 * k;
        const int8_t *slo = mode == Q8_ACT_I8X2 ? lo + r0 * k : nullptr;
        int32_t *ssums = sums + r0 * n * nb * words;
        hipError_t e;
        if (mma_serves(mode, n, k, r, wb, shi, slo, shi, false)) {
            e = q8::launch_mma_sums(mode, wb, n, k, r, shi, slo, ssums, st);
        } else {
            e = hipSuccess;
            for (int c0 = 0; c0 < r && e == hipSuccess; c0 += 8) {
                const int c = std::min(8, r - c0);
                e = q8::launch_gemv_sums(words, wb, n, k, c, shi + c0 * k, slo ? slo + c0 * k : nullptr,
                                         ssums + c0 * n * nb * words, n, st);
            }
        }
        if (e != hipSuccess) return Q8_E_HIP;
    }
    return Q8_OK;
}

const char *q8_status_name(int status) {
    switch (status) {
        case Q8_OK: return "Q8_OK";
        case Q8_E_NULL: return "Q8_E_NULL";
        case Q8_E_SHAPE: return "Q8_E_SHAPE";
        case Q8_E_ALIGN: return "Q8_E_ALIGN";
        case Q8_E_MODE: return "Q8_E_MODE";
        case Q8_E_ALIAS: return "Q8_E_ALIAS";
        case Q8_E_HIP: return "Q8_E_HIP";
        default: return "Q8_E_UNKNOWN";
    }
}

int q8_version(void) { return 100; }

}  // extern "C"
