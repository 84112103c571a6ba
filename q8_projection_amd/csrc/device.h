// device.h -- device-side building blocks of the Q8_0 projection kernels (gfx950).
//
// A Q8_0 weight is consumed exactly as a checkpoint stores it: 34-byte blocks,
// a binary16 scale then 32 int8 values (model::author page, description;
// spatial::streamed page, description: weights travel in their stored form).  Block g
// of the whole matrix (row-major, g = n * nb + b) starts at byte 34 g, so odd
// blocks start 2 bytes past a dword boundary.  Every lane loads the 9 dwords of
// the dword-aligned window at or before its block (36 bytes, never past the end
// of the matrix when the block count is even) and realigns the 8 quant dwords
// with one v_perm_b32 each.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q8 {

constexpr int kBlock = 32;
constexpr int kBlockBytes = 34;

// The 36-byte dword-aligned window of one block.
struct Window {
    uint32_t d[9];
};

// Byte offset of block g's window (dword-aligned, at or before the block).
__device__ __forceinline__ int64_t window_offset(int64_t g) { return (g * kBlockBytes) & ~int64_t(3); }

// Load block g's window with the default cache policy (for this access pattern
// the non-temporal hint measured slower).  Needs only dword alignment.
__device__ __forceinline__ void load_window(const uint8_t *__restrict__ w, int64_t g, Window &out) {
    const uint32_t *p = reinterpret_cast<const uint32_t *>(w + window_offset(g));
#pragma unroll
    for (int i = 0; i < 9; ++i) out.d[i] = p[i];
}

__device__ __forceinline__ void zero_window(Window &out) {
#pragma unroll
    for (int i = 0; i < 9; ++i) out.d[i] = 0u;
}

// v_perm_b32 selector that extracts quant dword j from window dwords (j, j+1):
// even blocks start at window byte 0, their quants at byte 2; odd blocks start at
// window byte 2, their quants at byte 4.
__device__ __forceinline__ uint32_t window_selector(int64_t g) {
    return (g & 1) ? 0x07060504u : 0x05040302u;
}

// Bit pattern of the block's binary16 scale.
__device__ __forceinline__ uint32_t window_scale_bits(const Window &w, int64_t g) {
    return (g & 1) ? (w.d[0] >> 16) : (w.d[0] & 0xffffu);
}

// The 32 int8 quants as 8 dwords (little-endian: byte i of dword j is q[4j + i]).
__device__ __forceinline__ void window_quants(const Window &w, uint32_t sel, uint32_t (&q)[8]) {
#pragma unroll
    for (int j = 0; j < 8; ++j) q[j] = __builtin_amdgcn_perm(w.d[j + 1], w.d[j], sel);
}

__device__ __forceinline__ float f16_bits_to_float(uint32_t bits) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits)));
}

// Exact int32 dot product of 32 int8 pairs: 8 chained v_dot4 (|sum| <= 32*127*127).
__device__ __forceinline__ int32_t dot32(const uint32_t (&q)[8], const uint32_t (&a)[8]) {
    int32_t acc = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j)
        acc = __builtin_amdgcn_sdot4(static_cast<int>(q[j]), static_cast<int>(a[j]), acc, false);
    return acc;
}

// Buffer loads here address ranges under 2^31 bytes.  An offset with bit 31 set
// is past every range, so the load returns zeros and touches no memory.
// oob_bit(ok) is 0 for an in-range lane and that bit otherwise: OR-ing it in is
// plain arithmetic, so the compiler has no select to turn into a branch
// around the load.
__device__ __forceinline__ uint32_t oob_bit(bool ok) { return static_cast<uint32_t>(!ok) << 31; }

// Order this wave's LDS writes before its later LDS reads, for data exchanged
// between lanes of the wave (no instruction is emitted: LDS operations of one
// wave are already in order; this stops the compiler from reusing values it
// loaded before the exchange).
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
}

// Workgroup barrier after this wave's LDS writes have already been waited for
// by the caller (an explicit s_waitcnt): the acquire fence keeps later LDS
// reads from being moved above the barrier or served from earlier loads.
__device__ __forceinline__ void workgroup_barrier_acquire_lds() {
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// One DPP move of a double (each 32-bit half moved with the same control).
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
    const uint64_t b = __builtin_bit_cast(uint64_t, v);
    const int lo = __builtin_amdgcn_update_dpp(0, static_cast<int>(b), CTRL, 0xf, 0xf, false);
    const int hi = __builtin_amdgcn_update_dpp(0, static_cast<int>(b >> 32), CTRL, 0xf, 0xf, false);
    return __builtin_bit_cast(double, (static_cast<uint64_t>(static_cast<uint32_t>(hi)) << 32) |
                                          static_cast<uint32_t>(lo));
}

__device__ __forceinline__ double readlane_f64(double v, int lane) {
    const uint64_t b = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = __builtin_amdgcn_readlane(static_cast<int>(b), lane);
    const uint32_t hi = __builtin_amdgcn_readlane(static_cast<int>(b >> 32), lane);
    return __builtin_bit_cast(double, (static_cast<uint64_t>(hi) << 32) | lo);
}

// Sum of a double over the 64 lanes of a wave, in a fixed order; every lane
// gets the total.  Within each 16-lane row: pairs, quads (quad_perm), halves
// (row_half_mirror), the row (row_mirror); then the four row sums read out of
// lanes 0, 16, 32, 48.  No LDS round trips.
__device__ __forceinline__ double wave_sum(double v) {
    v += dpp_f64<0xb1>(v);   // quad_perm [1,0,3,2]
    v += dpp_f64<0x4e>(v);   // quad_perm [2,3,0,1]
    v += dpp_f64<0x141>(v);  // row_half_mirror
    v += dpp_f64<0x140>(v);  // row_mirror
    return (readlane_f64(v, 0) + readlane_f64(v, 16)) + (readlane_f64(v, 32) + readlane_f64(v, 48));
}

}  // namespace q8
