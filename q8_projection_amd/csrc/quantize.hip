// quantize.hip -- Q8_0 weight quantization and int8 activation quantization.
//
// Activation quantization is the lane's int8 activation (codegen_cuda::lane
// page, description: the one-word form and the default two-word ~14-bit form;
// Modules, kernels: an activation quantized for its projection).  Weight
// quantization produces the Q8_0 blocks a checkpoint stores (model::author page,
// description).  Rounding is decided exactly as written: correctly rounded f32
// division, round half away from zero, a fused multiply-add for the two-word
// residual, and no other contraction.
#include "device.h"
#include "launch.h"

#pragma clang fp contract(off)

namespace q8 {
namespace {

constexpr int kThreads = 256;
constexpr int kLanesPerBlock = 8;  // 8 lanes x 4 values = one 32-value block

__device__ __forceinline__ int quant_clamped(float v) {
    float r = roundf(v);  // half away from zero
    r = r > 127.0f ? 127.0f : r;
    r = r < -127.0f ? -127.0f : r;
    return static_cast<int>(r);
}

__device__ __forceinline__ float group_max8(float v) {
#pragma unroll
    for (int off = 1; off < kLanesPerBlock; off <<= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}

__device__ __forceinline__ uint32_t pack4(int a, int b, int c, int d) {
    return (static_cast<uint32_t>(a) & 0xffu) | ((static_cast<uint32_t>(b) & 0xffu) << 8) |
           ((static_cast<uint32_t>(c) & 0xffu) << 16) | ((static_cast<uint32_t>(d) & 0xffu) << 24);
}

// One thread per 4 consecutive values; 8 threads per 32-value block.  x, hi and
// lo are contiguous [rows][k] with k a multiple of 32, so block t/8 covers values
// 32*(t/8) .. +31 of the flat array and its scale is scale[t/8].
template <int WORDS>
__global__ __launch_bounds__(kThreads) void quantize_act_kernel(const float *__restrict__ x,
                                                                int64_t nblocks, int8_t *__restrict__ hi,
                                                                int8_t *__restrict__ lo,
                                                                float *__restrict__ scale) {
    const int64_t t = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    const int64_t blk = t / kLanesPerBlock;
    const bool valid = blk < nblocks;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (valid) v = *reinterpret_cast<const float4 *>(x + t * 4);
    float amax = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
    amax = group_max8(amax);
    if (!valid) return;
    const float s = amax / 127.0f;
    const float vals[4] = {v.x, v.y, v.z, v.w};
    int h[4], l[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        h[i] = (s == 0.0f) ? 0 : quant_clamped(vals[i] / s);
        if (WORDS == 2) {
            const float resid = __builtin_fmaf(-s, static_cast<float>(h[i]), vals[i]);
            l[i] = (s == 0.0f) ? 0 : quant_clamped((resid * 128.0f) / s);
        }
    }
    *reinterpret_cast<uint32_t *>(hi + t * 4) = pack4(h[0], h[1], h[2], h[3]);
    if (WORDS == 2) *reinterpret_cast<uint32_t *>(lo + t * 4) = pack4(l[0], l[1], l[2], l[3]);
    if ((t % kLanesPerBlock) == 0) scale[blk] = s;
}

// Weight quantization, same thread layout; block g is written at byte 34 g
// (2-byte aligned), so stores are 16-bit.
__global__ __launch_bounds__(kThreads) void quantize_weights_kernel(const float *__restrict__ w,
                                                                    int64_t nblocks,
                                                                    uint8_t *__restrict__ blocks) {
    const int64_t t = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    const int64_t blk = t / kLanesPerBlock;
    const int part = static_cast<int>(t % kLanesPerBlock);
    const bool valid = blk < nblocks;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (valid) {
        const float *p = w + t * 4;
        v = make_float4(p[0], p[1], p[2], p[3]);
    }
    float amax = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
    amax = group_max8(amax);
    if (!valid) return;
    const float d32 = amax / 127.0f;
    const _Float16 h = static_cast<_Float16>(d32);  // round to nearest even
    const float dq = static_cast<float>(h);
    const float vals[4] = {v.x, v.y, v.z, v.w};
    int q[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) q[i] = (dq == 0.0f) ? 0 : quant_clamped(vals[i] / dq);
    uint8_t *dst = blocks + blk * kBlockBytes;
    uint16_t *dst16 = reinterpret_cast<uint16_t *>(dst + 2 + 4 * part);
    dst16[0] = static_cast<uint16_t>((q[0] & 0xff) | ((q[1] & 0xff) << 8));
    dst16[1] = static_cast<uint16_t>((q[2] & 0xff) | ((q[3] & 0xff) << 8));
    if (part == 0) *reinterpret_cast<uint16_t *>(dst) = __builtin_bit_cast(uint16_t, h);
}

}  // namespace

hipError_t launch_quantize_act(int words, const float *x, int64_t rows, int64_t k, int8_t *hi,
                               int8_t *lo, float *scale, hipStream_t stream) {
    const int64_t nblocks = rows * (k / kBlock);
    const int64_t threads = nblocks * kLanesPerBlock;
    const dim3 grid(static_cast<unsigned>((threads + kThreads - 1) / kThreads));
    if (words == 2)
        quantize_act_kernel<2><<<grid, kThreads, 0, stream>>>(x, nblocks, hi, lo, scale);
    else
        quantize_act_kernel<1><<<grid, kThreads, 0, stream>>>(x, nblocks, hi, lo, scale);
    return hipGetLastError();
}

hipError_t launch_quantize_weights(const float *w, int64_t n, int64_t k, uint8_t *blocks,
                                   hipStream_t stream) {
    const int64_t nblocks = n * (k / kBlock);
    const int64_t threads = nblocks * kLanesPerBlock;
    const dim3 grid(static_cast<unsigned>((threads + kThreads - 1) / kThreads));
    quantize_weights_kernel<<<grid, kThreads, 0, stream>>>(w, nblocks, blocks);
    return hipGetLastError();
}

}  // namespace q8
