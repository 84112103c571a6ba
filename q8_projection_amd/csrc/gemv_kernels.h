// gemv_kernels.h -- the projection for stacks of 1..8 activation rows: a wave64
// GEMV over Q8_0 weights.  Kernel templates and their launch logic; the
// translation units gemv*.hip instantiate them (one activation mode each, and
// the block-sum export), so that they compile in parallel.
//
// Each weight row is streamed from HBM once for the whole stack (codegen_cuda::
// lane page, description: a stacked step passes over each weight a single time;
// model::author page, Functions: decode_batch).  The pages' own kernel
// runs four output rows a (32-wide) warp (codegen_cuda::lane page, Modules,
// plan: rows_a_warp).  Here a 64-wide wave owns a group of MR output rows at a
// time.  Its lanes stride over the rows' 34-byte blocks, so one wave-wide load
// covers 64 consecutive blocks (2176 contiguous bytes).
//
// Resident kernels (the activation stack fits in LDS): the grid is persistent and
// each wave walks a sequence of items (row group, 64-block column).  A register
// ring keeps P items of weight windows in flight.  Weight windows are read with
// range-checked buffer loads: a lane or item outside the matrix reads zeros
// without touching memory and without a branch, so every item issues the same
// loads and the wait counts stay exact.  For the same reason the main loop
// holds no other vector-memory operation: each row's f64 total goes to LDS, and
// the residual add and the f32 store run after the loop.
//
// Tiled kernels (the stack is too large for LDS): the stack is staged in column
// tiles between barriers and each wave owns one row group.
//
// The activation stack (int8 words and block scales, or f32 values) is staged
// with direct-to-LDS loads.  Integer modes take exact int32 block sums with
// v_dot4; every block term is accumulated in f64 and each output is rounded once.
//
// Block-sum export (SUMS): the same kernel writes each block's exact int32 sums
// S_hi (and S_lo) to a caller buffer where the projection accumulates them, so
// the integer dot products of the kernel that serves a call can be checked bit
// for bit.
#pragma once

#include <algorithm>

#include "actquant.h"
#include "device.h"
#include "launch.h"

namespace q8 {

struct GemvArgs {
    const uint8_t *w;       // Q8_0 blocks [n][nb]
    const int8_t *hi;       // [rows][k]
    const int8_t *lo;       // [rows][k] (two-word)
    const float *scale;     // [rows][nb]
    const float *x;         // [rows][k] (f32 mode)
    const float *residual;  // [rows][n] or null
    float *y;               // [rows][n]
    int64_t n;              // weight rows of this launch
    int64_t ldy;            // row stride of y and residual (elements)
    int k;
    int nb;
    int kt;                 // columns per LDS tile (a multiple of 64); kt == k: resident
    int ntiles;
    int ub;                 // 64-block columns per tile
    int64_t num_groups;     // row groups of MR rows
    int32_t *argmax;        // one activation row: also write the arg-max of y here, or null
    uint32_t *argmax_work;  // its workspace: [0] a counter left at zero, then [grid][2] partials
    int32_t *sums;          // block-sum export: [rows][sums_ld][nb][words] int32, or null
    int64_t sums_ld;        // weight rows of the whole call (the export's row stride)
};

// Per activation mode (translation units gemv_f32.hip, gemv_i8.hip,
// gemv_i8x2.hip) and for the block-sum export (gemv_sums.hip).
hipError_t gemv_dispatch_f32(int rows, const GemvArgs &a, hipStream_t s);
hipError_t gemv_dispatch_i8(int rows, const GemvArgs &a, hipStream_t s);
hipError_t gemv_dispatch_i8x2(int rows, const GemvArgs &a, hipStream_t s);
hipError_t gemv_dispatch_sums(int words, int rows, const GemvArgs &a, hipStream_t s);

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kLdsBudget = 64 * 1024;     // LDS for the staged stack, per workgroup
constexpr int kOutPerWave = 128;          // f64 totals a wave may park in LDS
constexpr int kTiledMaxUb = 4;            // 64-block columns per tile in the tiled kernels
constexpr uint32_t kBufferDword3 = 0x00020000u;  // raw buffer resource, gfx9 family
constexpr uint32_t kOob = 0x80000000u;    // an offset past every range: reads return 0
constexpr int64_t kMaxStreamBytes = int64_t(1) << 30;  // weight bytes one resident launch streams
constexpr int kLoadsPerWindow = 3;       // buffer loads issue_item makes per window
constexpr int kLoadPolicy = 0;            // cache policy of the weight stream (default: measured fastest)

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------------ staging

// The activation stack is copied into LDS with gfx950's direct-to-LDS loads
// (global_load_lds_dwordx4 / _dword): the data never passes through VGPRs.  One
// wave-wide instruction moves one chunk (64 lanes x 16 or 4 bytes) to a
// wave-uniform LDS address; chunks are dealt round-robin to the workgroup's
// waves.  Callers wait for the copies (vmcnt) and then barrier.  The copies are
// inline assembly: the compiler does not track them, so it never adds waits for
// them on its own (every wait on them is the caller's explicit one), and the
// weight stream behind them is not drained before each LDS read.

typedef __attribute__((address_space(3))) void *lptr_t;

__device__ __forceinline__ uint32_t lds_address(const void *p) {
    return __builtin_amdgcn_readfirstlane(static_cast<uint32_t>((uintptr_t)(lptr_t)p));
}
__device__ __forceinline__ void lds_copy16(const void *src, uint32_t lds) {
    asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(lds) : "memory");
}
__device__ __forceinline__ void lds_copy4(const void *src, uint32_t lds) {
    asm volatile("global_load_lds_dword %0, off" ::"v"(src), "{m0}"(lds) : "memory");
}

// f32 stacks in LDS: the eight 16-byte granules of each 32-value block sit in
// the order j ^ (block & 7).  A lane reads its own block's granules, so lanes
// of one block apart are 128 bytes apart; in plain order the 16-byte reads of
// eight neighbouring lanes all fell on the same four banks.  Swizzled, they
// cover every bank.  The copies place it: a lane picks its source granule.
__host__ __device__ constexpr int f32_granule(int block, int j) { return j ^ (block & 7); }

// rows x bytes (bytes a multiple of 16) from src (row stride src_stride) to LDS
// dst (row stride dst_stride), 16 bytes per lane.  F32_SWIZZLE: the rows are
// f32 values (bytes a multiple of 128), stored in the order above.
template <bool F32_SWIZZLE = false>
__device__ __forceinline__ void dma_rows16(uint8_t *dst, int dst_stride, const uint8_t *src, int64_t src_stride,
                                           int rows, int bytes, int wave, int lane) {
    const int per_row = (bytes + 1023) / 1024;
    // a copy covers 1 KB = 8 whole blocks, so lane / 8 is the block's index mod 8
    const int from = F32_SWIZZLE ? (lane & ~7) + f32_granule(lane >> 3, lane & 7) : lane;
    for (int c = wave; c < rows * per_row; c += kWaves) {
        const int r = c / per_row, off = (c - r * per_row) * 1024;
        const uint32_t to = lds_address(dst + r * dst_stride + off);
        if (off + lane * 16 < bytes) lds_copy16(src + r * src_stride + off + from * 16, to);
    }
}

// rows x count f32 values from src (row stride src_stride floats) to LDS dst
// (row stride dst_stride floats), one dword per lane.
__device__ __forceinline__ void dma_rows4(float *dst, int dst_stride, const float *src, int64_t src_stride,
                                          int rows, int count, int wave, int lane) {
    const int per_row = (count + 63) / 64;
    for (int c = wave; c < rows * per_row; c += kWaves) {
        const int r = c / per_row, off = (c - r * per_row) * 64;
        const uint32_t to = lds_address(dst + r * dst_stride + off);
        if (off + lane < count) lds_copy4(src + r * src_stride + off + lane, to);
    }
}

// Wait until at most N of this wave's vector-memory operations are outstanding,
// then barrier.  The direct-to-LDS copies of a tile are issued before the N
// weight loads that follow them, and vmcnt retires in order, so after the wait
// this wave's copies have landed while its weight loads stay in flight; after
// the barrier every wave's copies have.  The explicit wait is the release.
template <int N>
__device__ __forceinline__ void staged_barrier() {
    static_assert(N >= 0 && N < 64, "vmcnt is six bits");
    // LDS stores of a stack quantized in place complete first (every copy is
    // inline assembly the compiler does not see, so this waits on LDS only)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    // s_waitcnt fields (gfx9): vmcnt[3:0] and [15:14], expcnt[6:4], lgkmcnt[11:8]
    __builtin_amdgcn_s_waitcnt((N & 0xf) | ((N >> 4) << 14) | 0x70 | 0xf00);
    workgroup_barrier_acquire_lds();
}

// Integer modes.  LDS: hi [R][kt] bytes, lo [R][kt] bytes (two-word), scales [R][kt/32] f32.
// SUMS: the block-sum export has no scales; they are not copied.
template <int R, int WORDS, bool SUMS = false>
__device__ __forceinline__ void stage_int(const GemvArgs &a, uint8_t *lds, int ti, int wave, int lane) {
    const int kt0 = ti * a.kt, ktc = min(a.kt, a.k - kt0);
    dma_rows16(lds, a.kt, reinterpret_cast<const uint8_t *>(a.hi) + kt0, a.k, R, ktc, wave, lane);
    if (WORDS == 2)
        dma_rows16(lds + R * a.kt, a.kt, reinterpret_cast<const uint8_t *>(a.lo) + kt0, a.k, R, ktc, wave, lane);
    if constexpr (!SUMS)
        dma_rows4(reinterpret_cast<float *>(lds + WORDS * R * a.kt), a.kt / kBlock, a.scale + kt0 / kBlock, a.nb,
                  R, ktc / kBlock, wave, lane);
}

// Integer modes with the stack given as f32 x: each workgroup quantizes the
// tile itself into the layout stage_int copies (the lane's activation
// quantization fused into its consumer; codegen_cuda::lane page, Modules,
// kernels: fused forms), bit for bit as the stand-alone quantizer does.  Eight
// lanes per 32-value block; a whole wave always takes part in a block's maximum.
template <int R, int WORDS>
__device__ __forceinline__ void stage_quant(const GemvArgs &a, uint8_t *lds, int ti) {
    const int kt0 = ti * a.kt, ktc = min(a.kt, a.k - kt0);
    const int nbt = ktc / kBlock;
    int8_t *lhi = reinterpret_cast<int8_t *>(lds);
    int8_t *llo = lhi + R * a.kt;
    float *ls = reinterpret_cast<float *>(lhi + WORDS * R * a.kt);
    const int total = R * nbt * kQuantLanes;
    for (int t0 = 0; t0 < total; t0 += kThreads) {
        const int t = t0 + threadIdx.x;
        const bool valid = t < total;
        const int blk = t / kQuantLanes, part = t % kQuantLanes;
        const int r = blk / nbt, b = blk - r * nbt;
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (valid) v = *reinterpret_cast<const float4 *>(a.x + static_cast<int64_t>(r) * a.k + kt0 + b * kBlock + 4 * part);
        uint32_t h4, l4;
        const float sc = quantize4<WORDS>(v, h4, l4);
        if (valid) {
            *reinterpret_cast<uint32_t *>(lhi + r * a.kt + b * kBlock + 4 * part) = h4;
            if (WORDS == 2) *reinterpret_cast<uint32_t *>(llo + r * a.kt + b * kBlock + 4 * part) = l4;
            if (part == 0) ls[r * (a.kt / kBlock) + b] = sc;
        }
    }
}

// f32 mode.  LDS: x [R][kt] f32.
template <int R>
__device__ __forceinline__ void stage_f32(const GemvArgs &a, uint8_t *lds, int ti, int wave, int lane) {
    const int kt0 = ti * a.kt, ktc = min(a.kt, a.k - kt0);
    dma_rows16<true>(lds, a.kt * 4, reinterpret_cast<const uint8_t *>(a.x + kt0), static_cast<int64_t>(a.k) * 4, R,
                     ktc * 4, wave, lane);
}

// ------------------------------------------------------------- weight windows

// One item: row group grp, tile ti, 64-block column u (lane's block bl = u*64 + lane).
struct Item {
    int64_t grp;
    int ti;
    int u;
};

// Load the item's MR windows with range-checked buffer loads.  `live` is false
// for ring refills past the wave's last item: every lane then reads zeros.
template <int MR>
__device__ __forceinline__ void issue_item(const GemvArgs &a, const Item &it, bool live, int lane,
                                           Window (&win)[MR]) {
    const int ktb = a.kt / kBlock;
    const int kb0 = it.ti * ktb;
    const int nbt = min(ktb, a.nb - kb0);
    const int bl = it.u * 64 + lane;
    const int64_t row0 = it.grp * MR;
    const int64_t left = a.n - row0;
    const int rows_here = live ? static_cast<int>(left < 0 ? 0 : (left > MR ? MR : left)) : 0;
    const uint8_t *base = rows_here > 0 ? a.w + row0 * a.nb * kBlockBytes : a.w;
    const uint32_t range = static_cast<uint32_t>(rows_here) * static_cast<uint32_t>(a.nb) * kBlockBytes;
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(base), 0, static_cast<int>(range), kBufferDword3);
#pragma unroll
    for (int m = 0; m < MR; ++m) {
        const bool ok = bl < nbt && m < rows_here;
        const uint32_t off =
            static_cast<uint32_t>(window_offset(static_cast<int64_t>(m) * a.nb + kb0 + bl)) | oob_bit(ok);
        const u32x4 d0 = __builtin_amdgcn_raw_buffer_load_b128(rsrc, off, 0, kLoadPolicy);
        const u32x4 d1 = __builtin_amdgcn_raw_buffer_load_b128(rsrc, off + 16, 0, kLoadPolicy);
        const uint32_t d2 = __builtin_amdgcn_raw_buffer_load_b32(rsrc, off + 32, 0, kLoadPolicy);
        win[m].d[0] = d0.x; win[m].d[1] = d0.y; win[m].d[2] = d0.z; win[m].d[3] = d0.w;
        win[m].d[4] = d1.x; win[m].d[5] = d1.y; win[m].d[6] = d1.z; win[m].d[7] = d1.w;
        win[m].d[8] = d2;
    }
}

// ------------------------------------------------------------------- compute

// Integer modes: acc[m][r] += d * s * T with T = S_hi (one-word) or
// 128 S_hi + S_lo (two-word; the 1/128 is applied to the total, exactly).
// SUMS: also write S_hi (and S_lo) of every block to the export buffer.
template <int R, int WORDS, int MR, bool SUMS = false>
__device__ __forceinline__ void compute_int_item(const GemvArgs &a, const uint8_t *lds, const Item &it, int lane,
                                                 const Window (&win)[MR], double (&acc)[MR][R]) {
    const int ktb = a.kt / kBlock;
    const int kb0 = it.ti * ktb;
    const int nbt = min(ktb, a.nb - kb0);
    const int bl = it.u * 64 + lane;
    if (bl >= nbt) return;
    const int8_t *lhi = reinterpret_cast<const int8_t *>(lds);
    const int8_t *llo = lhi + R * a.kt;
    const float *ls = reinterpret_cast<const float *>(lhi + WORDS * R * a.kt);
    // The block's parity is all the realignment needs: nb and kb0 are even, so
    // block (grp*MR + m, kb0 + bl) has the parity of bl.
    const uint32_t sel = window_selector(bl);
    uint32_t q[MR][8];
    double d[MR];
#pragma unroll
    for (int m = 0; m < MR; ++m) {
        window_quants(win[m], sel, q[m]);
        d[m] = static_cast<double>(f16_bits_to_float(window_scale_bits(win[m], bl)));
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
        const double s = static_cast<double>(ls[r * ktb + bl]);
#pragma unroll
        for (int m = 0; m < MR; ++m) {
            const int32_t sh = dot32(q[m], h);
            const int32_t sl = WORDS == 2 ? dot32(q[m], l) : 0;
            const int32_t t = WORDS == 2 ? sh * 128 + sl : sh;
            acc[m][r] += (d[m] * s) * static_cast<double>(t);
            if constexpr (SUMS) {
                const int64_t row = it.grp * MR + m;
                if (row < a.n) {
                    int32_t *o = a.sums + ((static_cast<int64_t>(r) * a.sums_ld + row) * a.nb + kb0 + bl) * WORDS;
                    o[0] = sh;
                    if (WORDS == 2) o[1] = sl;
                }
            }
        }
    }
}

// f32 mode: acc[0][r] += d * sum_j q_j x_j, every product and sum in f64.
template <int R, int MR>
__device__ __forceinline__ void compute_f64_item(const GemvArgs &a, const uint8_t *lds, const Item &it, int lane,
                                                 const Window (&win)[MR], double (&acc)[MR][R]) {
    static_assert(MR == 1, "the f32 mode runs one weight row a wave");
    const int ktb = a.kt / kBlock;
    const int kb0 = it.ti * ktb;
    const int nbt = min(ktb, a.nb - kb0);
    const int bl = it.u * 64 + lane;
    if (bl >= nbt) return;
    const float *lx = reinterpret_cast<const float *>(lds);
    uint32_t q[8];
    window_quants(win[0], window_selector(bl), q);
    const double d = static_cast<double>(f16_bits_to_float(window_scale_bits(win[0], bl)));
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const float4 *px = reinterpret_cast<const float4 *>(lx + r * a.kt + bl * kBlock);
        double p = 0.0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float4 xv = px[f32_granule(bl, j)];
            const uint32_t qw = q[j];
            p = __builtin_fma(static_cast<double>(static_cast<int8_t>(qw)), static_cast<double>(xv.x), p);
            p = __builtin_fma(static_cast<double>(static_cast<int8_t>(qw >> 8)), static_cast<double>(xv.y), p);
            p = __builtin_fma(static_cast<double>(static_cast<int8_t>(qw >> 16)), static_cast<double>(xv.z), p);
            p = __builtin_fma(static_cast<double>(static_cast<int8_t>(qw >> 24)), static_cast<double>(xv.w), p);
        }
        acc[0][r] += d * p;
    }
}

template <int R, int WORDS, int MR, bool SUMS = false>
__device__ __forceinline__ void compute_item(const GemvArgs &a, const uint8_t *lds, const Item &it, int lane,
                                             const Window (&win)[MR], double (&acc)[MR][R]) {
    static_assert(!SUMS || WORDS != 0, "the block-sum export is for the integer modes");
    if constexpr (WORDS == 0)
        compute_f64_item<R, MR>(a, lds, it, lane, win, acc);
    else
        compute_int_item<R, WORDS, MR, SUMS>(a, lds, it, lane, win, acc);
}

template <int R, int WORDS, bool SUMS = false>
__device__ __forceinline__ void stage_tile(const GemvArgs &a, uint8_t *lds, int ti, int wave, int lane) {
    if constexpr (WORDS == 0)
        stage_f32<R>(a, lds, ti, wave, lane);
    else if constexpr (SUMS)
        stage_int<R, WORDS, true>(a, lds, ti, wave, lane);
    else if (a.x)
        stage_quant<R, WORDS>(a, lds, ti);
    else
        stage_int<R, WORDS>(a, lds, ti, wave, lane);
}

// Output element (r, row): the f64 total plus the residual in f64, rounded once.
__device__ __forceinline__ float write_output(const GemvArgs &a, int r, int64_t row, double tot) {
    const int64_t o = static_cast<int64_t>(r) * a.ldy + row;
    const double res = a.residual ? static_cast<double>(a.residual[o]) : 0.0;
    const float v = static_cast<float>(tot + res);
    a.y[o] = v;
    return v;
}

// ----------------------------------------------------------------- arg-max

// The LM head closes a decode step by picking the next token (model::author
// page, Functions: head, decode_step): argmax_i y[i], the
// lowest i among equal maxima.  Fused into the GEMV epilogue: every workgroup
// reduces its rows to one (value, row) partial in the workspace; an agent-scope
// atomic counter tells the last workgroup to finish, which reduces the partials
// (a max with a fixed tie-break, so the order of arrival does not matter),
// writes the index and puts the counter back to zero for the next call.
__device__ __forceinline__ bool argmax_better(float v, int32_t i, float bv, int32_t bi) {
    return v > bv || (v == bv && i < bi);
}

__device__ __forceinline__ void argmax_wave(float &v, int32_t &i) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const float ov = __shfl_xor(v, off, 64);
        const int32_t oi = __shfl_xor(i, off, 64);
        if (argmax_better(ov, oi, v, i)) {
            v = ov;
            i = oi;
        }
    }
}

// Called by every thread of the workgroup, with this lane's best (value, row).
__device__ __forceinline__ void argmax_finish(const GemvArgs &a, float v, int32_t i, int wave, int lane) {
    __shared__ float wave_v[kWaves];
    __shared__ int32_t wave_i[kWaves];
    __shared__ int is_last;
    uint32_t *counter = a.argmax_work;
    uint32_t *part = a.argmax_work + 4;  // 16-byte header, then [grid][2]
    argmax_wave(v, i);
    if (lane == 0) {
        wave_v[wave] = v;
        wave_i[wave] = i;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        float bv = wave_v[0];
        int32_t bi = wave_i[0];
        for (int w = 1; w < kWaves; ++w)
            if (argmax_better(wave_v[w], wave_i[w], bv, bi)) {
                bv = wave_v[w];
                bi = wave_i[w];
            }
        // The partial goes out as one agent-scope atomic store, which is written
        // through this XCD's L2 to the device-coherent level, and it has
        // completed (vmcnt counts stores too) before the count is taken.  A
        // release/acquire pair on the counter would instead write back and
        // invalidate the whole L2 in every workgroup; on the 151936-row head
        // (512 workgroups) that cost 20 us.
        const uint64_t packed = (static_cast<uint64_t>(static_cast<uint32_t>(bi)) << 32) | __float_as_uint(bv);
        __hip_atomic_store(reinterpret_cast<uint64_t *>(part) + blockIdx.x, packed, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        const uint32_t done = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        is_last = done == gridDim.x - 1;
    }
    __syncthreads();
    if (!is_last) return;
    // Every other workgroup's partial had completed before its count, and all
    // counts are in: read them at agent scope too (past this XCD's L2).
    v = -__builtin_inff();
    i = INT32_MAX;
    for (uint32_t b = threadIdx.x; b < gridDim.x; b += blockDim.x) {
        const uint64_t packed = __hip_atomic_load(reinterpret_cast<const uint64_t *>(part) + b, __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT);
        const float pv = __uint_as_float(static_cast<uint32_t>(packed));
        const int32_t pi = static_cast<int32_t>(packed >> 32);
        if (argmax_better(pv, pi, v, i)) {
            v = pv;
            i = pi;
        }
    }
    argmax_wave(v, i);
    __syncthreads();  // every wave has read wave_v/wave_i of the first round
    if (lane == 0) {
        wave_v[wave] = v;
        wave_i[wave] = i;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        float bv = wave_v[0];
        int32_t bi = wave_i[0];
        for (int w = 1; w < kWaves; ++w)
            if (argmax_better(wave_v[w], wave_i[w], bv, bi)) {
                bv = wave_v[w];
                bi = wave_i[w];
            }
        *a.argmax = bi;
        __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // ready for the next call
    }
}

// Epilogue of the resident kernels: scale (1/128 in two-word mode, exact),
// residual, one rounding, store; then the arg-max if asked for (one row).
template <int R, int WORDS, int MR>
__device__ __forceinline__ void finish_rows(const GemvArgs &a, const double *totals, int G, int64_t gw,
                                            int64_t stride, int wave, int lane) {
    const double post = WORDS == 2 ? 1.0 / 128.0 : 1.0;
    float best = -__builtin_inff();
    int32_t best_row = INT32_MAX;
    for (int i = lane; i < G * MR * R; i += 64) {
        const int gi = i / (MR * R), m = (i / R) % MR, r = i % R;
        const int64_t row = (gw + static_cast<int64_t>(gi) * stride) * MR + m;
        if (row < a.n) {
            const float v = write_output(a, r, row, totals[i] * post);
            if (argmax_better(v, static_cast<int32_t>(row), best, best_row)) {
                best = v;
                best_row = static_cast<int32_t>(row);
            }
        }
    }
    if constexpr (R == 1 && MR == 1)
        if (a.argmax) argmax_finish(a, best, best_row, wave, lane);
}

__host__ __device__ inline size_t stack_bytes(int rows, int words, int kt) {
    return words == 0 ? static_cast<size_t>(rows) * kt * 4
                      : static_cast<size_t>(rows) * words * kt + static_cast<size_t>(rows) * (kt / kBlock) * 4;
}

// ------------------------------------------------------------ resident kernel

// The whole matrix as one range-checked buffer (the launcher keeps it under
// 2^31 bytes).  Offsets are byte offsets into it; kOob reads zeros.
struct WeightStream {
    __amdgpu_buffer_rsrc_t rsrc;
    uint32_t lane_part;  // this lane's window offset within a 64-block column: (lane*34) & ~3
    uint32_t row_bytes;  // nb * 34
};

template <int MR>
__device__ __forceinline__ void stream_item(const WeightStream &ws, uint32_t item_base, bool lane_ok,
                                            Window (&win)[MR]) {
#pragma unroll
    for (int m = 0; m < MR; ++m) {
        // item_base: byte offset of the item's first block in its group's first row,
        // or kOob for a dead refill (then every offset below stays out of range)
        const uint32_t off = (item_base + m * ws.row_bytes + ws.lane_part) | oob_bit(lane_ok);
        const u32x4 d0 = __builtin_amdgcn_raw_buffer_load_b128(ws.rsrc, off, 0, kLoadPolicy);
        const u32x4 d1 = __builtin_amdgcn_raw_buffer_load_b128(ws.rsrc, off + 16, 0, kLoadPolicy);
        const uint32_t d2 = __builtin_amdgcn_raw_buffer_load_b32(ws.rsrc, off + 32, 0, kLoadPolicy);
        win[m].d[0] = d0.x; win[m].d[1] = d0.y; win[m].d[2] = d0.z; win[m].d[3] = d0.w;
        win[m].d[4] = d1.x; win[m].d[5] = d1.y; win[m].d[6] = d1.z; win[m].d[7] = d1.w;
        win[m].d[8] = d2;
    }
}

// Position of a wave in its item sequence: group gi (the wave's gi-th row group)
// and 64-block column u.  Advanced one item at a time.
struct Cursor {
    int gi;
    int u;
    __device__ __forceinline__ void next(int ub) {
        if (++u == ub) {
            u = 0;
            ++gi;
        }
    }
};

// WORDS = 1 or 2 (integer modes) or 0 (f32 mode).  SUMS: export the block
// sums instead of writing y (every memory operation of the loop is the
// compiler's, so it orders the export's stores itself).
template <int R, int WORDS, int MR, int P, bool SUMS = false>
__global__ __launch_bounds__(kThreads) void gemv_resident_kernel(GemvArgs a) {
    extern __shared__ __align__(16) uint8_t lds[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t gw = static_cast<int64_t>(blockIdx.x) * kWaves + wave;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kWaves;
    const int G = gw < a.num_groups ? static_cast<int>((a.num_groups - gw + stride - 1) / stride) : 0;
    const int ub = a.ub;
    const int T = G * ub;
    // per-row totals parked until the pipeline has drained: [group][m][r] f64
    const size_t totals_at = (stack_bytes(R, WORDS, a.kt) + 15) & ~size_t(15);
    double *totals = reinterpret_cast<double *>(lds + totals_at) + wave * kOutPerWave;

    WeightStream ws;
    ws.row_bytes = static_cast<uint32_t>(a.nb) * kBlockBytes;
    ws.rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(a.w), 0,
                                                static_cast<int>(static_cast<uint32_t>(a.n) * ws.row_bytes),
                                                kBufferDword3);
    ws.lane_part = static_cast<uint32_t>(lane * kBlockBytes) & ~3u;
    const uint32_t group_bytes = ws.row_bytes * MR;
    const uint32_t grid_group_bytes = static_cast<uint32_t>(stride) * group_bytes;
    const uint32_t first_group_bytes = static_cast<uint32_t>(gw) * group_bytes;
    // byte offset of item (gi, u) in the matrix, or kOob past the wave's items
    auto item_base = [&](const Cursor &c) -> uint32_t {
        return c.gi < G ? first_group_bytes + c.gi * grid_group_bytes + c.u * (64 * kBlockBytes) : kOob;
    };
    auto lane_ok = [&](const Cursor &c) { return c.u * 64 + lane < a.nb; };

    // Prologue: stage the stack (L2), then put the first P items of weights (HBM)
    // in flight, and barrier once the stack has landed.
    stage_tile<R, WORDS, SUMS>(a, lds, 0, wave, lane);
    Window ring[P][MR];
    Cursor ahead{0, 0};
#pragma unroll
    for (int p = 0; p < P; ++p) {
        stream_item<MR>(ws, item_base(ahead), lane_ok(ahead), ring[p]);
        ahead.next(ub);
    }
    staged_barrier<P * MR * kLoadsPerWindow>();

    double acc[MR][R];
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int r = 0; r < R; ++r) acc[m][r] = 0.0;

    Cursor cur{0, 0};
    for (int t0 = 0; t0 < T; t0 += P) {
#pragma unroll
        for (int p = 0; p < P; ++p) {
            const Item it{gw + static_cast<int64_t>(cur.gi) * stride, 0, cur.u};
            compute_item<R, WORDS, MR, SUMS>(a, lds, it, lane, ring[p], acc);
            stream_item<MR>(ws, item_base(ahead), lane_ok(ahead), ring[p]);
            ahead.next(ub);
            if (cur.gi < G && cur.u == ub - 1) {
#pragma unroll
                for (int m = 0; m < MR; ++m)
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        const double tot = wave_sum(acc[m][r]);
                        acc[m][r] = 0.0;
                        if (lane == 0) totals[(cur.gi * MR + m) * R + r] = tot;
                    }
            }
            cur.next(ub);
        }
    }
    if constexpr (SUMS) return;
    wave_lds_sync();  // lane 0 parked the totals the whole wave reads now
    finish_rows<R, WORDS, MR>(a, totals, G, gw, stride, wave, lane);
}

// ---------------------------------------------------- resident kernel, LDS ring

// The same walk as gemv_resident_kernel, with the weight windows staged through
// a per-wave LDS ring instead of registers.  One item row (64 blocks, 2176
// contiguous bytes) arrives by three direct-to-LDS copies marked non-temporal:
// two of 1 KB (16 bytes per lane) and one of 256 bytes (4 bytes per lane, the
// first 128 the item's tail).  Contiguous, whole-line copies let the stream use
// the non-temporal policy that the 36-byte per-lane windows cannot.  Each lane
// then reads its block's 36-byte window from the slot.  The copies are inline
// assembly (the compiler would otherwise wait for all of them before every LDS
// read); their waits are explicit.  Needs 16-byte aligned rows (k a multiple
// of 256) and a 16-byte aligned matrix.
constexpr int kItemBytes = 64 * kBlockBytes;  // 2176
constexpr int kSlotBytes = 2304;              // 2048 + the 256-byte copy
constexpr int kCopiesPerItemRow = 3;

__device__ __forceinline__ void copy_nt16(__amdgpu_buffer_rsrc_t r, uint32_t lds, uint32_t off) {
    asm volatile("buffer_load_dwordx4 %0, %1, 0 offen nt lds" ::"v"(off), "s"(r), "{m0}"(lds) : "memory");
}
__device__ __forceinline__ void copy_nt4(__amdgpu_buffer_rsrc_t r, uint32_t lds, uint32_t off) {
    asm volatile("buffer_load_dword %0, %1, 0 offen nt lds" ::"v"(off), "s"(r), "{m0}"(lds) : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vm() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void wait_lds_reads() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

// Copy item rows [item_base + m * row_bytes, + item_len) into the slot at LDS
// address `slot`.  item_base is kOob for a dead refill: every copy then reads
// zeros (bit 31 stays set).
template <int MR>
__device__ __forceinline__ void copy_item(const WeightStream &ws, uint32_t item_base, uint32_t item_len, int lane,
                                          uint32_t slot) {
    const uint32_t o0 = 16 * lane, o1 = 1024 + 16 * lane, o2 = 2048 + 4 * lane;
#pragma unroll
    for (int m = 0; m < MR; ++m) {
        const uint32_t row = item_base + m * ws.row_bytes;
        copy_nt16(ws.rsrc, slot + m * kSlotBytes, (row + o0) | oob_bit(o0 < item_len));
        copy_nt16(ws.rsrc, slot + m * kSlotBytes + 1024, (row + o1) | oob_bit(o1 < item_len));
        copy_nt4(ws.rsrc, slot + m * kSlotBytes + 2048, (row + o2) | oob_bit(o2 < item_len));
    }
}

template <int MR>
__device__ __forceinline__ void read_item(const uint8_t *slot, uint32_t lane_part, Window (&win)[MR]) {
#pragma unroll
    for (int m = 0; m < MR; ++m) {
        const uint32_t *p = reinterpret_cast<const uint32_t *>(slot + m * kSlotBytes + lane_part);
#pragma unroll
        for (int i = 0; i < 9; ++i) win[m].d[i] = p[i];
    }
}

// ------------------------------------------------- stack staged item by item

// A copied stack (integer words and scales, or f32 values) is staged in parts:
// part u holds the stack's columns [2048u, 2048u + 2048) of every row, the
// columns of the 64-block item u.  Part u is copied just before the weights of
// item u, so the wait for an item's weights also covers its part; in the first
// pass over the columns the workgroup meets at a barrier before each item.  A
// wave's first item then waits for one part rather than for the whole stack,
// which every workgroup asks L2 for at once at the start.  The LDS row stride kt
// is rounded up to a multiple of 2048 columns, so a part never spills into the
// next row; lanes past k read zeros.
constexpr int kPartCols = 64 * kBlock;  // 2048

__device__ __forceinline__ void copy16(__amdgpu_buffer_rsrc_t r, uint32_t lds, uint32_t off) {
    asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(off), "s"(r), "{m0}"(lds) : "memory");
}
__device__ __forceinline__ void copy4(__amdgpu_buffer_rsrc_t r, uint32_t lds, uint32_t off) {
    asm volatile("buffer_load_dword %0, %1, 0 offen lds" ::"v"(off), "s"(r), "{m0}"(lds) : "memory");
}

struct StackStream {
    __amdgpu_buffer_rsrc_t hi, lo, scale;  // [R][k], [R][k], [R][nb]; f32 mode: hi covers x [R][k]
};

// Copies of one part: per row, 1 KB copies of the int8 words (two per word) and
// one 256-byte copy of the 64 block scales, or eight 1 KB copies of f32 values.
// They are dealt round-robin to the workgroup's waves; a share that runs past
// the last copy repeats an earlier one (the same bytes to the same place), so
// every wave issues kPerWave copies a part.
template <int R, int WORDS>
struct PartPlan {
    static constexpr int kPerRow = WORDS == 0 ? 8 : 2 * WORDS + 1;
    static constexpr int kCopies = R * kPerRow;
    static constexpr int kPerWave = (kCopies + kWaves - 1) / kWaves;
};

template <int R, int WORDS>
__device__ __forceinline__ void copy_part(const GemvArgs &a, const StackStream &ss, uint32_t stack_lds, int u,
                                          int wave, int lane) {
    using Plan = PartPlan<R, WORDS>;
#pragma unroll
    for (int i = 0; i < Plan::kPerWave; ++i) {
        const int c = (wave + i * kWaves) % Plan::kCopies;
        const int r = c / Plan::kPerRow, j = c % Plan::kPerRow;
        if constexpr (WORDS == 0) {
            // f32 values, 8 blocks a copy, in the swizzled granule order
            const int from = (lane & ~7) + f32_granule(lane >> 3, lane & 7);
            const uint32_t col = u * kPartCols + j * 256 + 4 * from;
            copy16(ss.hi, stack_lds + (r * a.kt + u * kPartCols + j * 256) * 4,
                   ((r * a.k + col) * 4) | oob_bit(col < static_cast<uint32_t>(a.k)));
        } else {
            if (j < 2 * WORDS) {
                const int word = j >> 1, half = j & 1;
                const uint32_t col = u * kPartCols + half * 1024 + 16 * lane;
                copy16(word == 0 ? ss.hi : ss.lo, stack_lds + (word * R + r) * a.kt + u * kPartCols + half * 1024,
                       (r * a.k + col) | oob_bit(col < static_cast<uint32_t>(a.k)));
            } else {
                const uint32_t blk = u * 64 + lane;
                copy4(ss.scale, stack_lds + WORDS * R * a.kt + (r * (a.kt / kBlock) + u * 64) * 4,
                      ((r * a.nb + blk) * 4) | oob_bit(blk < static_cast<uint32_t>(a.nb)));
            }
        }
    }
}

// s_waitcnt vmcnt(Base + e * Step) for a wave-uniform e in [0, E].
template <int Base, int Step, int E>
__device__ __forceinline__ void wait_vm_sel(int e) {
    if constexpr (E > 0) {
        if (e == E) {
            wait_vm<Base + E * Step>();
            return;
        }
        wait_vm_sel<Base, Step, E - 1>(e);
    } else {
        wait_vm<Base>();
    }
}

__host__ __device__ inline size_t ring_lds_offset(int rows, int words, int kt) {
    return ((stack_bytes(rows, words, kt) + 15) & ~size_t(15)) + static_cast<size_t>(kWaves) * kOutPerWave * 8;
}

// PROG: the stack is copied part by part (above); otherwise it is quantized
// here from f32 x, whole, before the first item.  SUMS (with PROG, integer
// modes): export the block sums instead of writing y; the stack's scales are
// not read (the export has none) and every export store is waited for before
// the next copy is counted.
template <int R, int WORDS, int MR, int P, bool PROG, bool SUMS = false>
__global__ __launch_bounds__(kThreads) void gemv_ring_kernel(GemvArgs a) {
    static_assert(!SUMS || (PROG && WORDS != 0), "the export runs on the copied integer stack");
    extern __shared__ __align__(16) uint8_t lds[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t gw = static_cast<int64_t>(blockIdx.x) * kWaves + wave;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kWaves;
    const int G = gw < a.num_groups ? static_cast<int>((a.num_groups - gw + stride - 1) / stride) : 0;
    const int ub = a.ub;
    const int T = G * ub;
    const size_t totals_at = (stack_bytes(R, WORDS, a.kt) + 15) & ~size_t(15);
    double *totals = reinterpret_cast<double *>(lds + totals_at) + wave * kOutPerWave;
    uint8_t *ring = lds + ring_lds_offset(R, WORDS, a.kt) + wave * (P * MR * kSlotBytes);
    const uint32_t ring_lds = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>((uintptr_t)(lptr_t)ring));

    WeightStream ws;
    ws.row_bytes = static_cast<uint32_t>(a.nb) * kBlockBytes;
    ws.rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(a.w), 0,
                                                static_cast<int>(static_cast<uint32_t>(a.n) * ws.row_bytes),
                                                kBufferDword3);
    ws.lane_part = static_cast<uint32_t>(lane * kBlockBytes) & ~3u;
    const uint32_t group_bytes = ws.row_bytes * MR;
    const uint32_t grid_group_bytes = static_cast<uint32_t>(stride) * group_bytes;
    const uint32_t first_group_bytes = static_cast<uint32_t>(gw) * group_bytes;
    auto item_base = [&](const Cursor &c) -> uint32_t {
        return c.gi < G ? first_group_bytes + c.gi * grid_group_bytes + c.u * kItemBytes : kOob;
    };
    auto item_len = [&](const Cursor &c) -> uint32_t {
        return static_cast<uint32_t>(min(64, a.nb - c.u * 64)) * kBlockBytes;
    };

    double acc[MR][R];
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int r = 0; r < R; ++r) acc[m][r] = 0.0;
    auto flush_row = [&](const Cursor &c) {
        if (c.gi < G && c.u == ub - 1) {
#pragma unroll
            for (int m = 0; m < MR; ++m)
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const double tot = wave_sum(acc[m][r]);
                    acc[m][r] = 0.0;
                    if (lane == 0) totals[(c.gi * MR + m) * R + r] = tot;
                }
        }
    };
    constexpr int kItemOps = MR * kCopiesPerItemRow;
    Cursor ahead{0, 0};
    Cursor cur{0, 0};
    if constexpr (PROG) {
        using Plan = PartPlan<R, WORDS>;
        static_assert(P * (kItemOps + Plan::kPerWave) < 64, "in-flight copies exceed the vmcnt range");
        StackStream ss;
        if constexpr (WORDS == 0) {
            ss.hi = __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(a.x), 0, R * a.k * 4, kBufferDword3);
            ss.lo = ss.scale = ss.hi;
        } else {
            ss.hi = __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t *>(a.hi), 0, R * a.k, kBufferDword3);
            ss.lo = WORDS == 2 ? __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t *>(a.lo), 0, R * a.k,
                                                                   kBufferDword3)
                               : ss.hi;
            // the export passes no scales: an empty range reads zeros, touching nothing
            ss.scale = SUMS ? __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t *>(a.hi), 0, 0, kBufferDword3)
                            : __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(a.scale), 0, R * a.nb * 4,
                                                                kBufferDword3);
        }
        const uint32_t stack_lds = lds_address(lds);
        // Item t's part (t < ub) goes out just before item t's weights.
        auto issue = [&](int t, uint32_t slot) {
            if (t < ub) copy_part<R, WORDS>(a, ss, stack_lds, t, wave, lane);
            copy_item<MR>(ws, item_base(ahead), item_len(ahead), lane, slot);
            ahead.next(ub);
        };
        // Item 0 (and its part) goes out alone first, about a quarter of a
        // microsecond ahead of the rest, so that the chip's first burst serves
        // every wave's first item before any second one (measured: 3-5% on
        // 14336x4096 and 4096x4096, no change at 4096x14336 or on the LM head;
        // longer gaps were slower).
#pragma unroll
        for (int p = 0; p < P; ++p) {
            if (p == 1) __builtin_amdgcn_s_sleep(10);  // 10 x 64 clocks
            issue(p, ring_lds + p * MR * kSlotBytes);
        }
        // Every wave, with rows or without, takes part in the first pass's
        // barriers.
        const int Tp = max(T, ub);
        for (int t0 = 0; t0 < Tp; t0 += P) {
#pragma unroll
            for (int p = 0; p < P; ++p) {
                const int t = t0 + p;
                // this item's copies (and its part) have landed; the later
                // items in flight carry parts while they are below ub
                wait_vm_sel<(P - 1) * kItemOps, Plan::kPerWave, P - 1>(min(max(ub - 1 - t, 0), P - 1));
                if (t < ub) {  // every wave's share of part t has landed
                    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
                    workgroup_barrier_acquire_lds();
                }
                Window win[MR];
                read_item<MR>(ring + p * MR * kSlotBytes, ws.lane_part, win);
                const Item it{gw + static_cast<int64_t>(cur.gi) * stride, 0, cur.u};
                compute_item<R, WORDS, MR, SUMS>(a, lds, it, lane, win, acc);
                // the export's stores have completed before later waits count copies
                if constexpr (SUMS) wait_vm<0>();
                wait_lds_reads();  // the slot is read before it is refilled
                issue(t + P, ring_lds + p * MR * kSlotBytes);
                flush_row(cur);
                cur.next(ub);
            }
        }
    } else {
        // The stack is quantized here from f32 x after the first copies go out
        // (its x loads are waited for by count, which then covers the copies
        // too, so the two latencies overlap), then one barrier.
#pragma unroll
        for (int p = 0; p < P; ++p) {
            copy_item<MR>(ws, item_base(ahead), item_len(ahead), lane, ring_lds + p * MR * kSlotBytes);
            ahead.next(ub);
        }
        stage_tile<R, WORDS>(a, lds, 0, wave, lane);
        staged_barrier<P * kItemOps>();
        for (int t0 = 0; t0 < T; t0 += P) {
#pragma unroll
            for (int p = 0; p < P; ++p) {
                wait_vm<(P - 1) * kItemOps>();  // this item's copies have landed
                Window win[MR];
                read_item<MR>(ring + p * MR * kSlotBytes, ws.lane_part, win);
                const Item it{gw + static_cast<int64_t>(cur.gi) * stride, 0, cur.u};
                compute_item<R, WORDS, MR>(a, lds, it, lane, win, acc);
                wait_lds_reads();  // the slot is read before it is refilled
                copy_item<MR>(ws, item_base(ahead), item_len(ahead), lane, ring_lds + p * MR * kSlotBytes);
                ahead.next(ub);
                flush_row(cur);
                cur.next(ub);
            }
        }
    }
    wait_vm<0>();  // the dead refills read nothing but still write the ring
    if constexpr (SUMS) return;
    wave_lds_sync();  // lane 0 parked the totals the whole wave reads now
    finish_rows<R, WORDS, MR>(a, totals, G, gw, stride, wave, lane);
}

// --------------------------------------------------------------- tiled kernel

// The stack is staged one column tile at a time; each wave owns one row group and
// keeps its (at most kTiledMaxUb) items of the tile in registers.
// SUMS: export the block sums instead of writing y; the export's stores are
// waited for before the next tile's copies are counted.
template <int R, int WORDS, int MR, bool SUMS = false>
__global__ __launch_bounds__(kThreads) void gemv_tiled_kernel(GemvArgs a) {
    extern __shared__ __align__(16) uint8_t lds[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t grp = static_cast<int64_t>(blockIdx.x) * kWaves + wave;
    double acc[MR][R];
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int r = 0; r < R; ++r) acc[m][r] = 0.0;
    for (int ti = 0; ti < a.ntiles; ++ti) {
        if (ti > 0) __syncthreads();  // every wave is done with the previous tile
        stage_tile<R, WORDS, SUMS>(a, lds, ti, wave, lane);
        Window win[kTiledMaxUb][MR];
#pragma unroll
        for (int u = 0; u < kTiledMaxUb; ++u)
            issue_item<MR>(a, Item{grp, ti, u}, u < a.ub && grp < a.num_groups, lane, win[u]);
        staged_barrier<kTiledMaxUb * MR * kLoadsPerWindow>();
#pragma unroll
        for (int u = 0; u < kTiledMaxUb; ++u)
            if (u < a.ub) compute_item<R, WORDS, MR, SUMS>(a, lds, Item{grp, ti, u}, lane, win[u], acc);
        if constexpr (SUMS) wait_vm<0>();
    }
    if constexpr (SUMS) return;
    const double post = WORDS == 2 ? 1.0 / 128.0 : 1.0;
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const double tot = wave_sum(acc[m][r]) * post;
            const int64_t row = grp * MR + m;
            if (lane == ((m * R + r) & 63) && row < a.n) write_output(a, r, row, tot);
        }
}

// ------------------------------------------------------------------- launchers

// Tile width (columns, a multiple of 64): the whole k when the staged stack fits
// the LDS budget, else k split into equal tiles that fit and hold at most
// kTiledMaxUb 64-block columns.
int tile_columns(int k, int rows, int words) {
    const int64_t per64 = static_cast<int64_t>(stack_bytes(rows, words, 64));
    int64_t kt_max = std::max<int64_t>(64, (kLdsBudget / per64) * 64);
    if (kt_max >= k) return k;
    kt_max = std::min<int64_t>(kt_max, static_cast<int64_t>(kTiledMaxUb) * 64 * kBlock);
    const int64_t ntiles = (k + kt_max - 1) / kt_max;
    return static_cast<int>(((k + ntiles - 1) / ntiles + 63) / 64 * 64);
}

constexpr int kWavesPerCu = 8;

// The LDS a ring launch needs, and whether the ring kernel serves the call
// (one tile, 16-byte aligned rows and matrix, two workgroups' LDS per CU).
template <int R, int WORDS, int MR, int P>
size_t ring_lds_bytes(int k) {
    const int kt_ring = (k + kPartCols - 1) / kPartCols * kPartCols;  // whole 2048-column parts
    return ring_lds_offset(R, WORDS, kt_ring) + static_cast<size_t>(kWaves) * P * MR * kSlotBytes;
}
template <int R, int WORDS, int MR, int P>
bool ring_serves(const GemvArgs &a) {
    const int64_t row_bytes = static_cast<int64_t>(a.nb) * kBlockBytes;
    const bool one_tile = tile_columns(a.k, R, WORDS) >= a.k;
    const bool aligned = (row_bytes % 16) == 0 && (reinterpret_cast<uintptr_t>(a.w) & 15) == 0;
    return one_tile && aligned &&
           ring_lds_bytes<R, WORDS, MR, P>(a.k) * 2 <= static_cast<size_t>(device_info().lds_per_block);
}

// SUMS: the block-sum export of the same call, from the kernel that projects it.
template <int R, int WORDS, int MR, int P, bool SUMS = false>
hipError_t run(GemvArgs a, hipStream_t stream) {
    a.kt = tile_columns(a.k, R, WORDS);
    a.ntiles = (a.k + a.kt - 1) / a.kt;
    a.ub = (a.kt / kBlock + 63) / 64;
    a.num_groups = (a.n + MR - 1) / MR;
    const size_t stack = stack_bytes(R, WORDS, a.kt);
    const int64_t row_bytes = static_cast<int64_t>(a.nb) * kBlockBytes;
    if (a.ntiles == 1 && a.n * row_bytes > kMaxStreamBytes) {
        // The resident kernel addresses the matrix as one buffer: run it on row
        // slices of at most kMaxStreamBytes.
        const int64_t slice = std::max<int64_t>(MR, (kMaxStreamBytes / row_bytes) / MR * MR);
        for (int64_t r0 = 0; r0 < a.n; r0 += slice) {
            GemvArgs s = a;
            s.w = a.w + r0 * row_bytes;
            s.n = std::min(slice, a.n - r0);
            s.y = a.y ? a.y + r0 : nullptr;
            s.residual = a.residual ? a.residual + r0 : nullptr;
            s.sums = a.sums ? a.sums + r0 * a.nb * (WORDS == 2 ? 2 : 1) : nullptr;
            if (hipError_t e = run<R, WORDS, MR, P, SUMS>(s, stream); e != hipSuccess) return e;
        }
        return hipSuccess;
    }
    if (a.ntiles == 1) {
        const DeviceInfo dev = device_info();
        // enough waves to fill the chip, and enough that none parks more than
        // kOutPerWave totals
        // the ring kernel stages the stack in whole 2048-column parts
        const int kt_ring = (a.k + kPartCols - 1) / kPartCols * kPartCols;
        const size_t ring_lds = ring_lds_bytes<R, WORDS, MR, P>(a.k);
        const size_t cu_lds = static_cast<size_t>(dev.lds_per_block);
        const bool ring = ring_serves<R, WORDS, MR, P>(a);
        // The f32 mode's f64 math leaves the SIMDs half idle at two waves each:
        // where three of its workgroups fit a CU it runs 12 waves a CU
        // (measured at 14336x4096: 17.6-18.7 -> 16.1-16.3 us; 16 waves were
        // slower than 12).  Not with the fused arg-max, whose workspace is
        // sized for the 8-wave grid.
        const int per_cu = (WORDS == 0 && ring && !a.argmax && ring_lds * 3 <= cu_lds) ? 12 : kWavesPerCu;
        const int64_t groups_cap = kOutPerWave / (MR * R);
        const int64_t min_waves = (a.num_groups + groups_cap - 1) / groups_cap;
        int64_t waves = std::min<int64_t>(a.num_groups, static_cast<int64_t>(dev.cus) * per_cu);
        waves = std::max<int64_t>(waves, min_waves);
        const int64_t grid = (waves + kWaves - 1) / kWaves;
        const size_t lds = ((stack + 15) & ~size_t(15)) + static_cast<size_t>(kWaves) * kOutPerWave * 8;
        if (ring) {
            GemvArgs b = a;
            b.kt = kt_ring;
            const dim3 g(static_cast<unsigned>(grid));
            if constexpr (SUMS)
                gemv_ring_kernel<R, WORDS, MR, P, true, true><<<g, kThreads, ring_lds, stream>>>(b);
            else if (WORDS != 0 && a.x != nullptr)
                gemv_ring_kernel<R, WORDS, MR, P, false><<<g, kThreads, ring_lds, stream>>>(b);
            else
                gemv_ring_kernel<R, WORDS, MR, P, true><<<g, kThreads, ring_lds, stream>>>(b);
        } else {
            gemv_resident_kernel<R, WORDS, MR, P, SUMS><<<dim3(static_cast<unsigned>(grid)), kThreads, lds, stream>>>(a);
        }
    } else {
        const int64_t grid = (a.num_groups + kWaves - 1) / kWaves;
        gemv_tiled_kernel<R, WORDS, MR, SUMS><<<dim3(static_cast<unsigned>(grid)), kThreads, stack, stream>>>(a);
    }
    return hipGetLastError();
}

// Kernel shape per stack height (rows per wave group MR, items in flight P).
template <int WORDS, bool SUMS = false>
hipError_t dispatch_int(int rows, const GemvArgs &a, hipStream_t s) {
    switch (rows) {
        case 1: return run<1, WORDS, 1, 2, SUMS>(a, s);
        case 2: return run<2, WORDS, 2, 4, SUMS>(a, s);
        case 3: return run<3, WORDS, 2, 4, SUMS>(a, s);
        case 4: return run<4, WORDS, 2, 4, SUMS>(a, s);
        case 5: return run<5, WORDS, 2, 2, SUMS>(a, s);
        case 6: return run<6, WORDS, 2, 2, SUMS>(a, s);
        case 7: return run<7, WORDS, 2, 2, SUMS>(a, s);
        default: return run<8, WORDS, 2, 2, SUMS>(a, s);
    }
}


}  // namespace
}  // namespace q8
