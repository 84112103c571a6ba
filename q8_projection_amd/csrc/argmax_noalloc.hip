// argmax_noalloc.hip -- the fused arg-max LM head for callers that cannot
// allocate: its workspace (a counter and one partial per workgroup) lives in a
// fixed device array of this library instead of a caller buffer.
//
// The array is a file-scope device variable, one copy per GPU, held until the
// process ends.  Host code never uses its name as an address (that is only a
// host-side stand-in): the device address is looked up once per device with
// hipGetSymbolAddress, with that device current, on the first call there, and
// kept; kernels get that address as an argument, as they get a caller's
// workspace.  Every call on a GPU shares its array: each call first clears the
// counter with a one-workgroup kernel on its own stream (no memset, so the pair
// can be captured into a graph), and two calls in flight on one GPU race.
#include <mutex>

#include "launch.h"

namespace {

constexpr int64_t kScratchBytes = 64 * 1024;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_lock;
void *g_scratch[kMaxDevices];  // device address of `scratch`, per device

// The workspace's 16-byte header (the arrival counter) back to zero.
__global__ void clear_header(uint32_t *header) {
    if (threadIdx.x < 4) header[threadIdx.x] = 0u;
}

}  // namespace

namespace q8 {

int64_t argmax_scratch_bytes() { return kScratchBytes; }

hipError_t argmax_scratch(void **out) {
    int dev = -1;
    if (hipError_t e = hipGetDevice(&dev); e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> guard(g_lock);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        if (hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)); e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return hipSuccess;
}

hipError_t launch_clear_argmax_header(void *workspace, hipStream_t stream) {
    clear_header<<<1, 64, 0, stream>>>(static_cast<uint32_t *>(workspace));
    return hipGetLastError();
}

}  // namespace q8
