// quantize.hip -- Q8_0 weight quantization and int8 activation quantization.
//
// Activation quantization is the lane's int8 activation (codegen_cuda::lane
// page, description: the one-word form and the default two-word ~14-bit form;
// Modules, kernels: an activation quantized for its projection).  Weight
// quantization produces the Q8_0 blocks a checkpoint stores (model::author page,
// description).  Rounding is decided exactly as written: correctly rounded f32
// division, round half away from zero, a fused multiply-add for the two-word
// residual, and no other contraction.
#include "actquant.h"
#include "device.h"
#include "launch.h"

#pragma clang fp contract(off)

namespace q8 {
namespace {

constexpr int kThreads = 256;
constexpr int kLanesPerBlock = kQuantLanes;  // 8 lanes x 4 values = one 32-value block

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
    uint32_t h4, l4;
    const float s = quantize4<WORDS>(v, h4, l4);  // all 8 lanes of the block take part
    if (!valid) return;
    *reinterpret_cast<uint32_t *>(hi + t * 4) = h4;
    if (WORDS == 2) *reinterpret_cast<uint32_t *>(lo + t * 4) = l4;
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
