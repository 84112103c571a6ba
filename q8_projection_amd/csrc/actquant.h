// actquant.h -- int8 block quantization of activations, shared by the
// stand-alone quantizer and the projections that quantize their own input.
//
// The lane's int8 activation forms (codegen_cuda::lane page, description: llama.cpp's
// one int8 word, and the default two-word ~14-bit form): per 32-value block,
// s = max|x| / 127 in f32, hi = rha(x / s) and, two-word, lo = rha((x - s*hi) * 128 / s)
// with the residual x - s*hi formed by one fused multiply-add.  Divisions are
// correctly rounded (the library is built with -fhip-fp32-correctly-rounded-divide-sqrt),
// rha is round half away from zero, an all-zero block gives zeros, and no other
// operation is contracted.  Both users call quantize4, so their bits agree.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q8 {

constexpr int kQuantLanes = 8;  // lanes per 32-value block, 4 values each

__device__ __forceinline__ int quant_clamped(float v) {
    float r = roundf(v);  // half away from zero
    r = r > 127.0f ? 127.0f : r;
    r = r < -127.0f ? -127.0f : r;
    return static_cast<int>(r);
}

// Maximum over the 8 consecutive lanes of a block (all 8 must call it).
__device__ __forceinline__ float group_max8(float v) {
#pragma unroll
    for (int off = 1; off < kQuantLanes; off <<= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}

__device__ __forceinline__ uint32_t pack4(int a, int b, int c, int d) {
    return (static_cast<uint32_t>(a) & 0xffu) | ((static_cast<uint32_t>(b) & 0xffu) << 8) |
           ((static_cast<uint32_t>(c) & 0xffu) << 16) | ((static_cast<uint32_t>(d) & 0xffu) << 24);
}

// Quantize this lane's 4 values of a block; the block's 8 lanes call it
// together (a lane with nothing to do passes zeros).  Returns the block scale;
// h4 / l4 are the packed words (l4 only for WORDS == 2).
template <int WORDS>
__device__ __forceinline__ float quantize4(float4 v, uint32_t &h4, uint32_t &l4) {
#pragma clang fp contract(off)
    float amax = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
    amax = group_max8(amax);
    const float s = amax / 127.0f;
    const float vals[4] = {v.x, v.y, v.z, v.w};
    int h[4], l[4] = {0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        h[i] = (s == 0.0f) ? 0 : quant_clamped(vals[i] / s);
        if (WORDS == 2) {
            const float resid = __builtin_fmaf(-s, static_cast<float>(h[i]), vals[i]);
            l[i] = (s == 0.0f) ? 0 : quant_clamped((resid * 128.0f) / s);
        }
    }
    h4 = pack4(h[0], h[1], h[2], h[3]);
    l4 = pack4(l[0], l[1], l[2], l[3]);
    return s;
}

}  // namespace q8
