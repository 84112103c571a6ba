// mfma.hip -- the projection for wide stacks of 9..64 activation rows (prefill
// chunks) on gfx950's int8 matrix cores.
//
// A prefill chunk stacks a block of prompt rows and every projection reads its
// weights once for the whole block (codegen_cuda::lane page, description;
// model::author page, Functions: prefill).  With 9..64 rows the product is a
// small dense contraction.  One Q8_0 block (32 columns) is exactly the K of one
// v_mfma_i32_32x32x32_i8, so the int32 result of each MFMA is the exact block dot
// product S[n][r] for a 32x32 tile.  It is rescaled by the block's two scales and
// accumulated in f64.  The rescale (three f64 VALU ops per tile element and block)
// is what bounds this kernel, alongside the weight stream.
//
// Roles: operand A = 32 weight rows (one 34-byte block per row and lane half),
// operand B = 32 activation rows.  In the result, lane l holds activation row
// l%32 and weight rows (v%4) + 8(v/4) + 4(l/32) in register v, so each lane's
// activation scale is one value per block.  The 32 weight scales are shared
// through a small LDS slot.  A workgroup owns one 32-row weight tile; its four
// waves each take a quarter of the blocks and are summed in a fixed order
// through LDS at the end.  Two-word activations take a second MFMA on the lo
// word and combine T = 128 S_hi + S_lo exactly in int32.
#include <algorithm>

#include "device.h"
#include "launch.h"

namespace q8 {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;    // the K split of one weight tile
constexpr int kTile = 32;                // weight rows (and activation rows) per MFMA tile
constexpr int kWavesPerSimd = 2;         // occupancy the register budget is held to
constexpr uint32_t kBufferDword3 = 0x00020000u;
constexpr int64_t kMaxStreamBytes = int64_t(1) << 30;

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct MfmaArgs {
    const uint8_t *w;
    const int8_t *hi;
    const int8_t *lo;
    const float *scale;
    const float *residual;
    float *y;
    int64_t n;     // weight rows of this launch
    int64_t ldy;   // row stride of y and residual
    int k;
    int nb;
    int rows;      // activation rows, 1..64
};

// Everything one lane loads for one block.
template <int RT, int WORDS>
struct Slot {
    uint32_t w[5];   // 20 window bytes: this lane half's 16 quants (and, in half 0, the scale)
    v4i h[RT];       // 16 hi bytes of activation row 32t + l%32
    v4i l[WORDS == 2 ? RT : 1];
    float s[RT];     // that row's block scale
};

struct Streams {
    __amdgpu_buffer_rsrc_t w, hi, lo, sc;
};

template <int RT, int WORDS>
__device__ __forceinline__ void load_block(const MfmaArgs &a, const Streams &st, int64_t tile0, int b, bool live,
                                           int lane, Slot<RT, WORDS> &sl) {
    const int half = lane >> 5;
    const int64_t row = tile0 + (lane & 31);
    // Window of block (row, b) (row * nb * 34 is a multiple of 4: nb is even).
    // Out of range lanes set bit 31, past every range: arithmetic, not a select,
    // so no load sits behind a branch.
    const uint32_t woff = (static_cast<uint32_t>(row * a.nb * kBlockBytes) +
                           ((static_cast<uint32_t>(b) * kBlockBytes) & ~3u) + 16u * half) |
                          oob_bit(live && row < a.n);
    const u32x4 w0 = __builtin_amdgcn_raw_buffer_load_b128(st.w, woff, 0, 0);
    const uint32_t w4 = __builtin_amdgcn_raw_buffer_load_b32(st.w, woff + 16, 0, 0);
    sl.w[0] = w0.x; sl.w[1] = w0.y; sl.w[2] = w0.z; sl.w[3] = w0.w; sl.w[4] = w4;
#pragma unroll
    for (int t = 0; t < RT; ++t) {
        const int r = t * kTile + (lane & 31);
        const uint32_t oob = oob_bit(live && r < a.rows);
        const uint32_t aoff = (static_cast<uint32_t>(r) * a.k + b * kBlock + 16 * half) | oob;
        sl.h[t] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(st.hi, aoff, 0, 0));
        if (WORDS == 2) sl.l[t] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(st.lo, aoff, 0, 0));
        const uint32_t soff = ((static_cast<uint32_t>(r) * a.nb + b) * 4u) | oob;
        sl.s[t] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(st.sc, soff, 0, 0));
    }
}

template <int RT, int WORDS>
__device__ __forceinline__ void compute_block(int b, int lane, const Slot<RT, WORDS> &sl, double *dslot,
                                              double (&acc)[RT][16]) {
    const int half = lane >> 5;
    // nb is even, so block (row, b) has the parity of b
    const uint32_t sel = (b & 1) ? 0x07060504u : 0x05040302u;
    v4i q;
    q.x = static_cast<int>(__builtin_amdgcn_perm(sl.w[1], sl.w[0], sel));
    q.y = static_cast<int>(__builtin_amdgcn_perm(sl.w[2], sl.w[1], sel));
    q.z = static_cast<int>(__builtin_amdgcn_perm(sl.w[3], sl.w[2], sel));
    q.w = static_cast<int>(__builtin_amdgcn_perm(sl.w[4], sl.w[3], sel));
    // half 0 holds the block's scale: share the tile's 32 scales through LDS
    const uint32_t dbits = (b & 1) ? (sl.w[0] >> 16) : (sl.w[0] & 0xffffu);
    if (half == 0) dslot[lane] = static_cast<double>(f16_bits_to_float(dbits));
    // Other lanes wrote the scales this lane reads: a wave-scope LDS fence, so
    // the reads below are not served from an earlier block's values.
    wave_lds_sync();
    v16i c[RT];
#pragma unroll
    for (int t = 0; t < RT; ++t) {
        const v16i zero = {};
        c[t] = __builtin_amdgcn_mfma_i32_32x32x32_i8(q, sl.h[t], zero, 0, 0, 0);
        if (WORDS == 2) {
            const v16i clo = __builtin_amdgcn_mfma_i32_32x32x32_i8(q, sl.l[t], zero, 0, 0, 0);
#pragma unroll
            for (int v = 0; v < 16; ++v) c[t][v] = c[t][v] * 128 + clo[v];
        }
    }
    // weight row of register v: (v%4) + 8(v/4) + 4*half -- four runs of 4 consecutive rows
    double d[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const double *src = dslot + 8 * i + 4 * half;
        d[4 * i + 0] = src[0];
        d[4 * i + 1] = src[1];
        d[4 * i + 2] = src[2];
        d[4 * i + 3] = src[3];
    }
#pragma unroll
    for (int t = 0; t < RT; ++t) {
        const double s = static_cast<double>(sl.s[t]);
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[t][v] += (d[v] * s) * static_cast<double>(c[t][v]);
    }
}

template <int RT, int WORDS, int P>
__global__ __launch_bounds__(kThreads, kWavesPerSimd) void mfma_kernel(MfmaArgs a) {
    __shared__ double dslots[kWaves][kTile];
    __shared__ double red[RT][16][64];   // one wave's partial tile, [t][v][lane]
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t tile0 = static_cast<int64_t>(blockIdx.x) * kTile;
    const int b0 = (wave * a.nb) / kWaves, b1 = ((wave + 1) * a.nb) / kWaves;
    const int T = b1 - b0;

    Streams st;
    const int64_t wrange = a.n * a.nb * kBlockBytes;
    st.w = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(a.w), 0, static_cast<int>(wrange), kBufferDword3);
    st.hi = __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t *>(a.hi), 0, a.rows * a.k, kBufferDword3);
    st.lo = __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t *>(WORDS == 2 ? a.lo : a.hi), 0, a.rows * a.k,
                                              kBufferDword3);
    st.sc = __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(a.scale), 0, a.rows * a.nb * 4, kBufferDword3);

    double acc[RT][16];
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[t][v] = 0.0;

    Slot<RT, WORDS> ring[P];
#pragma unroll
    for (int p = 0; p < P; ++p) {
        load_block<RT, WORDS>(a, st, tile0, b0 + p, p < T, lane, ring[p]);
        __builtin_amdgcn_sched_barrier(0);  // slots issue in order, oldest first
    }
    for (int t0 = 0; t0 < T; t0 += P) {
#pragma unroll
        for (int p = 0; p < P; ++p) {
            const int t = t0 + p;
            compute_block<RT, WORDS>(b0 + t, lane, ring[p], dslots[wave], acc);
            // keep each refill's loads together and after the block that freed
            // its slot, so the wait for a slot counts only the younger slots
            __builtin_amdgcn_sched_barrier(0);
            load_block<RT, WORDS>(a, st, tile0, b0 + t + P, t + P < T, lane, ring[p]);
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // Sum the four K quarters in a fixed order: ((q3 + q2) + q1) + q0.
    for (int q = kWaves - 1; q >= 1; --q) {
        if (wave == q) {
#pragma unroll
            for (int t = 0; t < RT; ++t)
#pragma unroll
                for (int v = 0; v < 16; ++v) red[t][v][lane] = acc[t][v];
        }
        __syncthreads();
        if (wave == q - 1) {
#pragma unroll
            for (int t = 0; t < RT; ++t)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[t][v] = red[t][v][lane] + acc[t][v];
        }
        __syncthreads();
    }
    if (wave == 0) {
#pragma unroll
        for (int t = 0; t < RT; ++t)
#pragma unroll
            for (int v = 0; v < 16; ++v) red[t][v][lane] = acc[t][v];
    }
    __syncthreads();
    // Coalesced epilogue: element (r, j) of the tile (weight row tile0 + j) sits in
    // register v = (j%4) + 4(j/8) of lane (r%32) + 32 ((j/4)%2).
    const double post = WORDS == 2 ? 1.0 / 128.0 : 1.0;
    for (int e = threadIdx.x; e < RT * kTile * kTile; e += kThreads) {
        const int r = e / kTile, j = e % kTile;
        const int64_t row = tile0 + j;
        if (r >= a.rows || row >= a.n) continue;
        const int t = r / kTile, src_lane = (r % kTile) + 32 * ((j / 4) % 2), v = (j % 4) + 4 * (j / 8);
        const int64_t o = static_cast<int64_t>(r) * a.ldy + row;
        const double res = a.residual ? static_cast<double>(a.residual[o]) : 0.0;
        a.y[o] = static_cast<float>(red[t][v][src_lane] * post + res);
    }
}

template <int RT, int WORDS, int P>
hipError_t run(MfmaArgs a, hipStream_t stream) {
    const int64_t row_bytes = static_cast<int64_t>(a.nb) * kBlockBytes;
    if (a.n * row_bytes > kMaxStreamBytes) {
        // weight offsets are 32-bit: run row slices of at most kMaxStreamBytes
        const int64_t slice = std::max<int64_t>(kTile, (kMaxStreamBytes / row_bytes) / kTile * kTile);
        for (int64_t r0 = 0; r0 < a.n; r0 += slice) {
            MfmaArgs s = a;
            s.w = a.w + r0 * row_bytes;
            s.n = std::min(slice, a.n - r0);
            s.y = a.y + r0;
            s.residual = a.residual ? a.residual + r0 : nullptr;
            if (hipError_t e = run<RT, WORDS, P>(s, stream); e != hipSuccess) return e;
        }
        return hipSuccess;
    }
    const int64_t grid = (a.n + kTile - 1) / kTile;
    mfma_kernel<RT, WORDS, P><<<dim3(static_cast<unsigned>(grid)), kThreads, 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace

bool mfma_supports(int mode, int rows) { return (mode == 1 || mode == 2) && rows > 8 && rows <= 64; }

hipError_t launch_mfma(int mode, const uint8_t *w, int64_t n, int64_t k, int rows, const int8_t *hi,
                       const int8_t *lo, const float *scale, const float *residual, float *y,
                       hipStream_t stream) {
    MfmaArgs a{};
    a.w = w;
    a.hi = hi;
    a.lo = lo;
    a.scale = scale;
    a.residual = residual;
    a.y = y;
    a.n = n;
    a.ldy = n;
    a.k = static_cast<int>(k);
    a.nb = static_cast<int>(k / kBlock);
    a.rows = rows;
    if (mode == 2) return rows > kTile ? run<2, 2, 2>(a, stream) : run<1, 2, 3>(a, stream);
    return rows > kTile ? run<2, 1, 2>(a, stream) : run<1, 1, 4>(a, stream);
}

}  // namespace q8
