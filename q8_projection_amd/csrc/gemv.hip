// gemv.hip -- the projection for stacks of 1..8 activation rows: wave64 GEMV
// over Q8_0 weights.
//
// Each weight row is streamed from HBM once for the whole stack (codegen_cuda::
// lane page, description: every projection reads its weights once for the
// block; model::author page, Functions: decode_batch).  The pages' own kernel
// runs four output rows a (32-wide) warp (codegen_cuda::lane page, Modules,
// plan: rows_a_warp); here a 64-wide wave owns MR output rows and its lanes
// stride over the rows' 34-byte blocks, so one wave-wide load instruction covers
// 64 consecutive blocks (2176 contiguous bytes).  The activation stack (int8
// words and block scales, or f32 values) is staged once per workgroup in LDS and
// read back per block.  Integer modes take exact int32 block sums with v_dot4;
// every block term is accumulated in f64 and each output is rounded once.
#include <algorithm>

#include "device.h"
#include "launch.h"

namespace q8 {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

struct GemvArgs {
    const uint8_t *w;       // Q8_0 blocks [n][nb]
    const int8_t *hi;       // [rows][k]
    const int8_t *lo;       // [rows][k] (two-word)
    const float *scale;     // [rows][nb]
    const float *x;         // [rows][k] (f32 mode)
    const float *residual;  // [rows][n] or null
    float *y;               // [rows][n]
    int64_t n;
    int k;
    int nb;
    int kt;                 // columns per LDS tile (multiple of 256)
    int64_t num_groups;     // row groups of kWaves * MR rows
};

// ---------------------------------------------------------------- integer modes

// LDS tile layout: hi [R][kt] bytes, lo [R][kt] bytes (two-word), then the block
// scales [R][kt/32] as f64 (divided by 128 in two-word mode, exact).
template <int R, int WORDS>
__device__ __forceinline__ void stage_int_tile(const GemvArgs &a, uint8_t *lds, int kt0, int ktc) {
    const int tid = threadIdx.x;
    const int vec_per_row = ktc / 16;
    int8_t *lhi = reinterpret_cast<int8_t *>(lds);
    int8_t *llo = lhi + R * a.kt;
    double *ls = reinterpret_cast<double *>(lhi + WORDS * R * a.kt);
    for (int i = tid; i < R * vec_per_row; i += kThreads) {
        const int r = i / vec_per_row, c = (i % vec_per_row) * 16;
        *reinterpret_cast<uint4 *>(lhi + r * a.kt + c) =
            *reinterpret_cast<const uint4 *>(a.hi + static_cast<int64_t>(r) * a.k + kt0 + c);
        if (WORDS == 2)
            *reinterpret_cast<uint4 *>(llo + r * a.kt + c) =
                *reinterpret_cast<const uint4 *>(a.lo + static_cast<int64_t>(r) * a.k + kt0 + c);
    }
    const int tbk = ktc / kBlock, kb0 = kt0 / kBlock, ktb = a.kt / kBlock;
    for (int i = tid; i < R * tbk; i += kThreads) {
        const int r = i / tbk, b = i % tbk;
        const double s = static_cast<double>(a.scale[static_cast<int64_t>(r) * a.nb + kb0 + b]);
        ls[r * ktb + b] = (WORDS == 2) ? s * (1.0 / 128.0) : s;
    }
}

template <int R, int WORDS, int MR, int U>
__global__ __launch_bounds__(kThreads) void gemv_int_kernel(GemvArgs a) {
    extern __shared__ __align__(16) uint8_t lds[];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int8_t *lhi = reinterpret_cast<const int8_t *>(lds);
    const int8_t *llo = lhi + R * a.kt;
    const double *ls = reinterpret_cast<const double *>(lhi + WORDS * R * a.kt);
    const int ktb = a.kt / kBlock;
    const bool resident = a.kt >= a.k;
    if (resident) {
        stage_int_tile<R, WORDS>(a, lds, 0, a.k);
        __syncthreads();
    }
    for (int64_t grp = blockIdx.x; grp < a.num_groups; grp += gridDim.x) {
        const int64_t n0 = (grp * kWaves + wave) * MR;
        double acc[MR][R];
#pragma unroll
        for (int m = 0; m < MR; ++m)
#pragma unroll
            for (int r = 0; r < R; ++r) acc[m][r] = 0.0;

        for (int kt0 = 0; kt0 < a.k; kt0 += a.kt) {
            const int ktc = min(a.kt, a.k - kt0);
            if (!resident) {
                __syncthreads();
                stage_int_tile<R, WORDS>(a, lds, kt0, ktc);
                __syncthreads();
            }
            const int tbk = ktc / kBlock, kb0 = kt0 / kBlock;
            for (int bl0 = 0; bl0 < tbk; bl0 += 64 * U) {
                Window win[U][MR];
#pragma unroll
                for (int u = 0; u < U; ++u)
#pragma unroll
                    for (int m = 0; m < MR; ++m) {
                        const int bl = bl0 + 64 * u + lane;
                        if (bl < tbk && n0 + m < a.n)
                            load_window(a.w, (n0 + m) * a.nb + kb0 + bl, win[u][m]);
                        else
                            zero_window(win[u][m]);
                    }
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int bl = bl0 + 64 * u + lane;
                    if (bl >= tbk) continue;
                    uint32_t q[MR][8];
                    double d[MR];
#pragma unroll
                    for (int m = 0; m < MR; ++m) {
                        const int64_t g = (n0 + m) * a.nb + kb0 + bl;
                        window_quants(win[u][m], window_selector(g), q[m]);
                        d[m] = static_cast<double>(f16_bits_to_float(window_scale_bits(win[u][m], g)));
                    }
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        uint32_t h[8], l[8];
                        const uint4 *ph = reinterpret_cast<const uint4 *>(lhi + r * a.kt + bl * kBlock);
                        const uint4 h0 = ph[0], h1 = ph[1];
                        h[0] = h0.x; h[1] = h0.y; h[2] = h0.z; h[3] = h0.w;
                        h[4] = h1.x; h[5] = h1.y; h[6] = h1.z; h[7] = h1.w;
                        if (WORDS == 2) {
                            const uint4 *pl = reinterpret_cast<const uint4 *>(llo + r * a.kt + bl * kBlock);
                            const uint4 l0 = pl[0], l1 = pl[1];
                            l[0] = l0.x; l[1] = l0.y; l[2] = l0.z; l[3] = l0.w;
                            l[4] = l1.x; l[5] = l1.y; l[6] = l1.z; l[7] = l1.w;
                        }
                        const double s = ls[r * ktb + bl];
#pragma unroll
                        for (int m = 0; m < MR; ++m) {
                            int32_t t = dot32(q[m], h);
                            if (WORDS == 2) t = t * 128 + dot32(q[m], l);
                            acc[m][r] += (d[m] * s) * static_cast<double>(t);
                        }
                    }
                }
            }
        }
#pragma unroll
        for (int m = 0; m < MR; ++m)
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const double tot = wave_sum(acc[m][r]);
                const int64_t nn = n0 + m;
                if (lane == ((m * R + r) & 63) && nn < a.n) {
                    const int64_t o = static_cast<int64_t>(r) * a.n + nn;
                    const double res = a.residual ? static_cast<double>(a.residual[o]) : 0.0;
                    a.y[o] = static_cast<float>(tot + res);
                }
            }
    }
}

// ------------------------------------------------------------------- f32 mode

// LDS tile: x [R][kt] f32.  Every product q*x and every sum is f64.
template <int R>
__device__ __forceinline__ void stage_f32_tile(const GemvArgs &a, float *lds, int kt0, int ktc) {
    const int vec_per_row = ktc / 4;
    for (int i = threadIdx.x; i < R * vec_per_row; i += kThreads) {
        const int r = i / vec_per_row, c = (i % vec_per_row) * 4;
        *reinterpret_cast<float4 *>(lds + r * a.kt + c) =
            *reinterpret_cast<const float4 *>(a.x + static_cast<int64_t>(r) * a.k + kt0 + c);
    }
}

template <int R, int U>
__global__ __launch_bounds__(kThreads) void gemv_f64_kernel(GemvArgs a) {
    extern __shared__ __align__(16) uint8_t lds_raw[];
    float *lx = reinterpret_cast<float *>(lds_raw);
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const bool resident = a.kt >= a.k;
    if (resident) {
        stage_f32_tile<R>(a, lx, 0, a.k);
        __syncthreads();
    }
    for (int64_t grp = blockIdx.x; grp < a.num_groups; grp += gridDim.x) {
        const int64_t nn = grp * kWaves + wave;  // one output row per wave
        double acc[R];
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r] = 0.0;
        for (int kt0 = 0; kt0 < a.k; kt0 += a.kt) {
            const int ktc = min(a.kt, a.k - kt0);
            if (!resident) {
                __syncthreads();
                stage_f32_tile<R>(a, lx, kt0, ktc);
                __syncthreads();
            }
            const int tbk = ktc / kBlock, kb0 = kt0 / kBlock;
            for (int bl0 = 0; bl0 < tbk; bl0 += 64 * U) {
                Window win[U];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int bl = bl0 + 64 * u + lane;
                    if (bl < tbk && nn < a.n)
                        load_window(a.w, nn * a.nb + kb0 + bl, win[u]);
                    else
                        zero_window(win[u]);
                }
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int bl = bl0 + 64 * u + lane;
                    if (bl >= tbk) continue;
                    const int64_t g = nn * a.nb + kb0 + bl;
                    uint32_t q[8];
                    window_quants(win[u], window_selector(g), q);
                    const double d = static_cast<double>(f16_bits_to_float(window_scale_bits(win[u], g)));
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        const float4 *px = reinterpret_cast<const float4 *>(lx + r * a.kt + bl * kBlock);
                        double p = 0.0;
#pragma unroll
                        for (int j = 0; j < 8; ++j) {
                            const float4 xv = px[j];
                            const uint32_t qw = q[j];
                            p = __builtin_fma(static_cast<double>(static_cast<int8_t>(qw)), static_cast<double>(xv.x), p);
                            p = __builtin_fma(static_cast<double>(static_cast<int8_t>(qw >> 8)), static_cast<double>(xv.y), p);
                            p = __builtin_fma(static_cast<double>(static_cast<int8_t>(qw >> 16)), static_cast<double>(xv.z), p);
                            p = __builtin_fma(static_cast<double>(static_cast<int8_t>(qw >> 24)), static_cast<double>(xv.w), p);
                        }
                        acc[r] += d * p;
                    }
                }
            }
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const double tot = wave_sum(acc[r]);
            if (lane == r && nn < a.n) {
                const int64_t o = static_cast<int64_t>(r) * a.n + nn;
                const double res = a.residual ? static_cast<double>(a.residual[o]) : 0.0;
                a.y[o] = static_cast<float>(tot + res);
            }
        }
    }
}

// ------------------------------------------------------------------- launchers

constexpr int kLdsBudget = 64 * 1024;  // per workgroup; leaves room for 2 workgroups a CU

int round_down_256(int64_t v) { return static_cast<int>((v / 256) * 256); }

template <int R, int WORDS, int MR, int U>
hipError_t run_int(GemvArgs a, hipStream_t stream) {
    const int64_t per_col_num = static_cast<int64_t>(R) * WORDS * 32 + R * 8;  // bytes per 32 columns
    int kt = round_down_256(static_cast<int64_t>(kLdsBudget) * 32 / per_col_num);
    if (kt >= a.k) kt = a.k;
    a.kt = kt;
    const size_t lds = static_cast<size_t>(R) * WORDS * kt + static_cast<size_t>(R) * (kt / kBlock) * 8;
    a.num_groups = (a.n + kWaves * MR - 1) / (kWaves * MR);
    const DeviceInfo dev = device_info();
    int64_t grid = a.num_groups;
    if (kt >= a.k) {
        const int64_t per_cu = std::max<int64_t>(1, std::min<int64_t>(8, (160 * 1024) / std::max<size_t>(lds, 1)));
        grid = std::min<int64_t>(grid, per_cu * dev.cus);
    }
    gemv_int_kernel<R, WORDS, MR, U><<<dim3(static_cast<unsigned>(grid)), kThreads, lds, stream>>>(a);
    return hipGetLastError();
}

template <int R, int U>
hipError_t run_f64(GemvArgs a, hipStream_t stream) {
    int kt = round_down_256(static_cast<int64_t>(kLdsBudget) / (4 * R));
    if (kt >= a.k) kt = a.k;
    a.kt = kt;
    const size_t lds = static_cast<size_t>(R) * kt * 4;
    a.num_groups = (a.n + kWaves - 1) / kWaves;
    const DeviceInfo dev = device_info();
    int64_t grid = a.num_groups;
    if (kt >= a.k) {
        const int64_t per_cu = std::max<int64_t>(1, std::min<int64_t>(8, (160 * 1024) / std::max<size_t>(lds, 1)));
        grid = std::min<int64_t>(grid, per_cu * dev.cus);
    }
    gemv_f64_kernel<R, U><<<dim3(static_cast<unsigned>(grid)), kThreads, lds, stream>>>(a);
    return hipGetLastError();
}

template <int WORDS>
hipError_t dispatch_int(int rows, const GemvArgs &a, hipStream_t s) {
    switch (rows) {
        case 1: return run_int<1, WORDS, 1, 4>(a, s);
        case 2: return run_int<2, WORDS, 2, 2>(a, s);
        case 3: return run_int<3, WORDS, 2, 2>(a, s);
        case 4: return run_int<4, WORDS, 2, 1>(a, s);
        case 5: return run_int<5, WORDS, 2, 1>(a, s);
        case 6: return run_int<6, WORDS, 2, 1>(a, s);
        case 7: return run_int<7, WORDS, 2, 1>(a, s);
        default: return run_int<8, WORDS, 2, 1>(a, s);
    }
}

hipError_t dispatch_f64(int rows, const GemvArgs &a, hipStream_t s) {
    switch (rows) {
        case 1: return run_f64<1, 2>(a, s);
        case 2: return run_f64<2, 2>(a, s);
        case 3: return run_f64<3, 1>(a, s);
        case 4: return run_f64<4, 1>(a, s);
        case 5: return run_f64<5, 1>(a, s);
        case 6: return run_f64<6, 1>(a, s);
        case 7: return run_f64<7, 1>(a, s);
        default: return run_f64<8, 1>(a, s);
    }
}

}  // namespace

hipError_t launch_gemv(int mode, const uint8_t *w, int64_t n, int64_t k, int rows, const int8_t *hi,
                       const int8_t *lo, const float *scale, const float *x, const float *residual,
                       float *y, hipStream_t stream) {
    GemvArgs a{};
    a.w = w;
    a.hi = hi;
    a.lo = lo;
    a.scale = scale;
    a.x = x;
    a.residual = residual;
    a.y = y;
    a.n = n;
    a.k = static_cast<int>(k);
    a.nb = static_cast<int>(k / kBlock);
    if (mode == 0) return dispatch_f64(rows, a, stream);
    if (mode == 2) return dispatch_int<2>(rows, a, stream);
    return dispatch_int<1>(rows, a, stream);
}

}  // namespace q8
