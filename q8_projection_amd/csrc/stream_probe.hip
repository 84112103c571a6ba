// stream_probe.hip -- libq8probe.so: a bare streaming read, the measured
// ceiling the projection kernels are compared with.  Not part of the
// projection library: only the benchmark loads it.
//
// One launch reads a device buffer once, start to end, in 2 KB items dealt
// round-robin to every wave of a persistent grid, exactly as the GEMV streams
// weight rows: direct-to-LDS buffer loads of 1 KB (64 lanes x 16 contiguous
// bytes, non-temporal), a ring of P items in flight per wave, each item waited
// for before its ring slot is refilled.  Nothing is computed, so the launch's
// time is what this memory system takes to deliver those bytes to the CUs in
// this form, fixed costs (launch, ramp, tail) included.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kItemBytes = 2048;
constexpr uint32_t kBufferDword3 = 0x00020000u;
constexpr uint32_t kOob = 0x80000000u;

__device__ __forceinline__ void copy_nt16(__amdgpu_buffer_rsrc_t r, uint32_t lds, uint32_t off) {
    asm volatile("buffer_load_dwordx4 %0, %1, 0 offen nt lds" ::"v"(off), "s"(r), "{m0}"(lds) : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vm() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Item i's two copies into ring slot `slot` (item offsets past the end carry
// the out-of-range bit: they read nothing).
__device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t r, uint32_t slot, uint32_t item, uint32_t nitems,
                                      int lane) {
    const uint32_t base = item < nitems ? item * kItemBytes : kOob;
    copy_nt16(r, slot, (base + 16 * lane) | (base & kOob));
    copy_nt16(r, slot + 1024, (base + 1024 + 16 * lane) | (base & kOob));
}

template <int P>
__global__ __launch_bounds__(kThreads) void stream_kernel(const uint8_t *buf, uint32_t nitems) {
    static_assert(2 * P <= 63, "in-flight copies within the vmcnt range");
    extern __shared__ __align__(16) uint8_t lds[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t gw = blockIdx.x * kWaves + wave;
    const uint32_t stride = gridDim.x * kWaves;
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(buf), 0, nitems * kItemBytes, kBufferDword3);
    const uint32_t ring = __builtin_amdgcn_readfirstlane(
        static_cast<uint32_t>((uintptr_t)(__attribute__((address_space(3))) uint8_t *)(lds + wave * P * kItemBytes)));
    const uint32_t mine = gw < nitems ? (nitems - gw + stride - 1) / stride : 0;
#pragma unroll
    for (int p = 0; p < P; ++p) issue(r, ring + p * kItemBytes, gw + p * stride, nitems, lane);
    for (uint32_t i = 0; i < mine; i += P) {
#pragma unroll
        for (int p = 0; p < P; ++p) {
            wait_vm<2 * (P - 1)>();  // item i + p has landed; refill its slot
            issue(r, ring + p * kItemBytes, gw + (i + p + P) * stride, nitems, lane);
        }
    }
    wait_vm<0>();
}

template <int P>
hipError_t launch(const uint8_t *buf, uint32_t nitems, int waves_per_cu, hipStream_t s) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                                                hipSuccess || cus <= 0)
        cus = 256;
    const int64_t waves = static_cast<int64_t>(cus) * waves_per_cu;
    const unsigned grid = static_cast<unsigned>((waves + kWaves - 1) / kWaves);
    stream_kernel<P><<<grid, kThreads, kWaves * P * kItemBytes, s>>>(buf, nitems);
    return hipGetLastError();
}

}  // namespace

extern "C" {

// Read `bytes` bytes of device memory at `buf` once.  bytes: a positive
// multiple of 2048 below 2^31; buf 16-byte aligned; ring: items in flight per
// wave (2, 4 or 8); waves_per_cu: 4..16.  Returns 0, -1 for bad arguments (no
// launch), or the HIP error of the launch.
int q8probe_stream(const void *buf, int64_t bytes, int ring, int waves_per_cu, void *stream) {
    if (!buf || bytes <= 0 || bytes % kItemBytes != 0 || bytes >= (int64_t(1) << 31)) return -1;
    if ((reinterpret_cast<uintptr_t>(buf) & 15) != 0 || waves_per_cu < 4 || waves_per_cu > 16) return -1;
    const uint8_t *b = static_cast<const uint8_t *>(buf);
    const uint32_t nitems = static_cast<uint32_t>(bytes / kItemBytes);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    switch (ring) {
        case 2: return launch<2>(b, nitems, waves_per_cu, s);
        case 4: return launch<4>(b, nitems, waves_per_cu, s);
        case 8: return launch<8>(b, nitems, waves_per_cu, s);
        default: return -1;
    }
}

}  // extern "C"
