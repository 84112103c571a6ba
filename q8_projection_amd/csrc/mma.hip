// mma.hip -- the projection for stacks of 2..64 activation rows on gfx950's
// int8 matrix cores, with every operand staged through an LDS ring.
//
// Batched decode and prefill chunks run the same projection over a stack of
// rows, reading each weight row once for the whole stack (codegen_cuda::lane
// page, description; model::author page, Functions: decode_batch, prefill).
//
// Work split.  A workgroup owns a contiguous range of at most RT*16 weight rows
// and walks K in chunks of 8 Q8_0 blocks (256 columns).  For every chunk it
// copies the range's weight bytes (272 contiguous bytes per row), the chunk of
// the activation words and the activation block scales into one slot of an LDS
// ring.  The copies are direct-to-LDS buffer loads: each instruction moves
// 1 KB, every lane 16 contiguous bytes, so HBM sees whole contiguous runs and
// no VGPR holds staged data.  The four waves of the workgroup issue the copies
// together and split the chunk's blocks for the math; one barrier per chunk
// hands a ring slot from the copies to the MFMAs, and the copies run
// kDepth - 1 chunks ahead.
//
// Math.  v_mfma_i32_16x16x32_i8 takes one block per instruction: operand A is
// 16 activation columns, operand B 16 weight rows, both 32 int8 along K, and the
// result is their 16x16 exact int32 block sums.  Lane l supplies column (or
// row) l%16, bytes 8(l/16)..8(l/16)+7 of the block, and receives columns
// 4(l/16)..4(l/16)+3 of weight row l%16.  In the two-word mode the 16 columns of
// a tile are the hi and lo words of 8 activation rows, ordered so that each lane
// receives both words of two rows: T = 128 S_hi + S_lo is formed exactly in
// int32.  Every block term (d * s) * T is accumulated in f64; at the end the
// four waves' partials are added in a fixed order and each output is rounded
// once to f32.
//
// The copies are issued with inline assembly on purpose: the compiler cannot
// tell ring slots apart and would otherwise wait for every outstanding copy
// before each LDS read.  The waits on the copies are explicit (vmcnt) and the
// barrier carries release/acquire fences for the LDS reads.
#include <algorithm>

#include "device.h"
#include "launch.h"

namespace q8 {
namespace {

#pragma clang fp contract(off)

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kChunkBlocks = 8;                            // blocks per chunk
constexpr int kRowChunk = kChunkBlocks * kBlockBytes;      // 272 bytes of one weight row
constexpr int kRowGranules = kRowChunk / 16;               // 17
constexpr int kActChunk = kChunkBlocks * kBlock;           // 256 activation bytes per row and word
constexpr int kCopyBytes = 1024;                           // one copy instruction: 64 lanes x 16 B
constexpr int kRingBudget = 144 * 1024;
constexpr int kMaxDepth = 12;
constexpr uint32_t kBufferDword3 = 0x00020000u;
constexpr uint32_t kOob = 0x80000000u;

typedef int v4i __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) uint8_t *lds_ptr_t;

// Sizes of one ring slot and of the ring, per instantiation.
//   RT: 16-row weight tiles per workgroup; AT: 16-column activation tiles.
template <int RT, int AT, int WORDS>
struct Layout {
    static constexpr int kRows = RT * 16;                      // weight rows a workgroup may own
    static constexpr int kActRows = AT * 16 / WORDS;           // activation rows the tiles hold
    static constexpr int kWCopies = (kRows * kRowGranules + 63) / 64;
    static constexpr int kACopies = AT * 4;                    // 16 columns x 256 B per tile
    static constexpr int kSCopies = (kActRows * 2 + 63) / 64;  // 8 f32 scales (2 granules) per row
    static constexpr int kCopies = kWCopies + kACopies + kSCopies;
    static constexpr int kPerWave = (kCopies + kWaves - 1) / kWaves;
    static constexpr int kSlotBytes = kPerWave * kWaves * kCopyBytes;  // tail copies are dummies
    static constexpr int kAOff = kWCopies * kCopyBytes;
    static constexpr int kSOff = kAOff + kACopies * kCopyBytes;
    static constexpr int kDepth = std::min(kMaxDepth, kRingBudget / kSlotBytes);
    static constexpr int kVals = WORDS == 2 ? 2 : 4;           // f64 accumulators per lane and tile pair
    static constexpr int kRedBytes = kWaves * RT * AT * kVals * 64 * 8;
    static constexpr int kLdsBytes = std::max(kDepth * kSlotBytes, kRedBytes);
    static_assert(kDepth >= 3, "the ring needs at least three slots");
    static_assert(kPerWave * (kDepth - 2) <= 63, "outstanding copies exceed the vmcnt range");
};

struct MmaArgs {
    const uint8_t *w;        // Q8_0 blocks [n][nb]
    const int8_t *hi;        // [rows][k]
    const int8_t *lo;        // [rows][k] (two-word)
    const float *scale;      // [rows][nb]
    const float *residual;   // [rows][ldy] or null
    float *y;                // [rows][ldy]
    int64_t ldy;
    uint32_t n;              // weight rows of this launch
    uint32_t k;
    uint32_t nb;
    uint32_t row_bytes;      // nb * 34
    uint32_t w_bytes;        // n * row_bytes (< 2^31)
    int rows;                // activation rows (<= kActRows)
    int rows_per_wg;
    int nchunks;             // nb / 8
};

struct Rsrcs {
    __amdgpu_buffer_rsrc_t w, hi, lo, s;
};

// One direct-to-LDS copy: lane i's 16 bytes at buffer offset `off` land at LDS
// address lds + 16 i.  An offset with bit 31 set reads zeros and touches no memory.
__device__ __forceinline__ void copy16(__amdgpu_buffer_rsrc_t r, uint32_t lds, uint32_t off) {
    asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(off), "s"(r), "{m0}"(lds) : "memory");
}

template <int N>
__device__ __forceinline__ void wait_copies() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Hand a ring slot over: this wave's LDS reads are complete (release) and the
// other waves' copies, already waited for with vmcnt, are visible (acquire).
__device__ __forceinline__ void ring_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// LDS column slot of activation column m of a tile.  Two-word: columns
// 4g+0..4g+3 are (hi, lo) of row 2g and (hi, lo) of row 2g+1; slots 0..7 hold
// hi rows 0..7 and slots 8..15 lo rows 0..7, so each copy instruction (four
// slots) reads one word array.  One-word: slot = column = row.
template <int WORDS>
__device__ __forceinline__ int act_slot(int m) {
    if constexpr (WORDS == 2)
        return ((m & 1) << 3) + ((m >> 2) << 1) + ((m >> 1) & 1);
    else
        return m;
}

// Copies of chunk c into the slot at LDS address `slot`.  Every wave issues
// exactly kPerWave copies (tail copies read nothing), so the vmcnt waits are
// exact.  Layout of a slot:
//   [0, kAOff)           weight rows, row-major, 272 bytes each (17 granules)
//   [kAOff, kSOff)       activation tiles: 16 column slots x 256 bytes, the
//                        16-byte granules of slot s XOR-permuted by s
//   [kSOff, ...)         activation scales, [row][8] f32
template <int RT, int AT, int WORDS>
__device__ __forceinline__ void issue_chunk(const MmaArgs &a, const Rsrcs &rs, uint32_t slot, int c, int wave,
                                            int lane, uint32_t r0, int rcount) {
    using L = Layout<RT, AT, WORDS>;
    const bool chunk_ok = c < a.nchunks;
#pragma unroll
    for (int u = 0; u < L::kPerWave; ++u) {
        const int i = wave + kWaves * u;  // wave-uniform copy index
        __amdgpu_buffer_rsrc_t r = rs.w;
        uint32_t off = kOob;
        if (i < L::kWCopies) {
            const int g = i * 64 + lane;
            const int row = g / kRowGranules;
            const int part = g - row * kRowGranules;
            const bool ok = chunk_ok && row < rcount;
            off = ((r0 + row) * a.row_bytes + c * kRowChunk + 16 * part) | oob_bit(ok);
        } else if (i < L::kWCopies + L::kACopies) {
            const int ia = i - L::kWCopies;
            const int t = ia >> 2;
            const int s = ((ia & 3) << 2) + (lane >> 4);  // column slot
            const int g = (lane & 15) ^ s;                // granule of the row's 256 chunk bytes
            int row;
            if constexpr (WORDS == 2) {
                row = t * 8 + (s & 7);
                r = (ia & 2) ? rs.lo : rs.hi;
            } else {
                row = t * 16 + s;
                r = rs.hi;
            }
            const bool ok = chunk_ok && row < a.rows;
            off = (static_cast<uint32_t>(row) * a.k + c * kActChunk + 16 * g) | oob_bit(ok);
        } else if (i < L::kCopies) {
            const int g = (i - L::kWCopies - L::kACopies) * 64 + lane;
            const int row = g >> 1;
            const bool ok = chunk_ok && row < a.rows;
            r = rs.s;
            off = (static_cast<uint32_t>(row) * a.nb * 4 + c * (kChunkBlocks * 4) + 16 * (g & 1)) | oob_bit(ok);
        }
        copy16(r, slot + i * kCopyBytes, off);
    }
}

// The math of one chunk for this wave: blocks wave and wave + 4 of the slot.
template <int RT, int AT, int WORDS>
__device__ __forceinline__ void compute_chunk(const uint8_t *slot, int wave, int lane,
                                              double (&acc)[RT][AT][Layout<RT, AT, WORDS>::kVals]) {
    using L = Layout<RT, AT, WORDS>;
    const int q = lane >> 4;   // operand k-quarter; result column group
    const int c16 = lane & 15; // operand column (A) / weight row (B and result)
    const int as = act_slot<WORDS>(c16);
#pragma unroll
    for (int jj = 0; jj < kChunkBlocks / kWaves; ++jj) {
        const int j = wave + kWaves * jj;  // wave-uniform block of the chunk
        long aop[AT];
        double s[AT][L::kVals];
#pragma unroll
        for (int t = 0; t < AT; ++t) {
            const uint8_t *pa = slot + L::kAOff + t * 4096 + as * 256 + ((((j << 1) + (q >> 1)) ^ as) << 4) + ((q & 1) << 3);
            aop[t] = *reinterpret_cast<const long *>(pa);
            const float *ps = reinterpret_cast<const float *>(slot + L::kSOff);
#pragma unroll
            for (int v = 0; v < L::kVals; ++v) {
                const int row = WORDS == 2 ? t * 8 + 2 * q + v : t * 16 + 4 * q + v;
                s[t][v] = static_cast<double>(ps[row * kChunkBlocks + j]);
            }
        }
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const uint8_t *prow = slot + (rt * 16 + c16) * kRowChunk;
            const int boff = j * kBlockBytes + 2 + 8 * q;  // first quant byte of this lane's operand
            const uint32_t *pw = reinterpret_cast<const uint32_t *>(prow + (boff & ~3));
            const uint32_t w0 = pw[0], w1 = pw[1], w2 = pw[2];
            const uint32_t sel = (boff & 2) ? 0x05040302u : 0x03020100u;
            const uint32_t lo32 = __builtin_amdgcn_perm(w1, w0, sel);
            const uint32_t hi32 = __builtin_amdgcn_perm(w2, w1, sel);
            const long bop = static_cast<long>((static_cast<uint64_t>(hi32) << 32) | lo32);
            const uint16_t dbits = *reinterpret_cast<const uint16_t *>(prow + j * kBlockBytes);
            const double d = static_cast<double>(f16_bits_to_float(dbits));
#pragma unroll
            for (int t = 0; t < AT; ++t) {
                const v4i dsum = __builtin_amdgcn_mfma_i32_16x16x32_i8(aop[t], bop, v4i{0, 0, 0, 0}, 0, 0, 0);
                if constexpr (WORDS == 2) {
                    const int t0 = dsum[0] * 128 + dsum[1];
                    const int t1 = dsum[2] * 128 + dsum[3];
                    acc[rt][t][0] = __builtin_fma(d * s[t][0], static_cast<double>(t0), acc[rt][t][0]);
                    acc[rt][t][1] = __builtin_fma(d * s[t][1], static_cast<double>(t1), acc[rt][t][1]);
                } else {
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        acc[rt][t][v] = __builtin_fma(d * s[t][v], static_cast<double>(dsum[v]), acc[rt][t][v]);
                }
            }
        }
    }
}

template <int RT, int AT, int WORDS>
__global__ __launch_bounds__(kThreads, 1) void mma_kernel(MmaArgs a) {
    using L = Layout<RT, AT, WORDS>;
    extern __shared__ __align__(16) uint8_t smem[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t r0 = blockIdx.x * static_cast<uint32_t>(a.rows_per_wg);
    const int rcount = static_cast<int>(min(static_cast<uint32_t>(a.rows_per_wg), a.n - r0));

    Rsrcs rs;
    rs.w = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(a.w), 0, a.w_bytes, kBufferDword3);
    const uint32_t act_bytes = static_cast<uint32_t>(a.rows) * a.k;
    rs.hi = __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t *>(a.hi), 0, act_bytes, kBufferDword3);
    rs.lo = WORDS == 2 ? __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t *>(a.lo), 0, act_bytes, kBufferDword3)
                       : rs.hi;
    rs.s = __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(a.scale), 0,
                                             static_cast<uint32_t>(a.rows) * a.nb * 4, kBufferDword3);

    const uint32_t base = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>((uintptr_t)(lds_ptr_t)smem));

    double acc[RT][AT][L::kVals];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int t = 0; t < AT; ++t)
#pragma unroll
            for (int v = 0; v < L::kVals; ++v) acc[rt][t][v] = 0.0;

    // Prologue: chunks 0 .. kDepth-2 in flight.
#pragma unroll
    for (int c = 0; c < L::kDepth - 1; ++c)
        issue_chunk<RT, AT, WORDS>(a, rs, base + c * L::kSlotBytes, c, wave, lane, r0, rcount);

    int cur = 0;                 // slot of chunk c
    int nxt = L::kDepth - 1;     // slot of chunk c + kDepth - 1
    for (int c = 0; c < a.nchunks; ++c) {
        wait_copies<L::kPerWave * (L::kDepth - 2)>();  // this wave's copies of chunk c have landed
        ring_barrier();                                // everyone's have; slot nxt is free
        issue_chunk<RT, AT, WORDS>(a, rs, base + nxt * L::kSlotBytes, c + L::kDepth - 1, wave, lane, r0, rcount);
        compute_chunk<RT, AT, WORDS>(smem + cur * L::kSlotBytes, wave, lane, acc);
        cur = cur + 1 == L::kDepth ? 0 : cur + 1;
        nxt = nxt + 1 == L::kDepth ? 0 : nxt + 1;
    }
    wait_copies<0>();  // the trailing copies read nothing but still write the ring
    ring_barrier();

    // Partials of the four waves, summed in a fixed order.
    double *red = reinterpret_cast<double *>(smem);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int t = 0; t < AT; ++t)
#pragma unroll
            for (int v = 0; v < L::kVals; ++v)
                red[(((wave * RT + rt) * AT + t) * L::kVals + v) * 64 + lane] = acc[rt][t][v];
    ring_barrier();

    const double post = WORDS == 2 ? 1.0 / 128.0 : 1.0;
    const int q = lane >> 4;
    const int c16 = lane & 15;
    for (int p = wave; p < RT * AT; p += kWaves) {
        const int rt = p / AT, t = p - (p / AT) * AT;
        const int row = rt * 16 + c16;
        if (row >= rcount) continue;
        const uint32_t n = r0 + row;
#pragma unroll
        for (int v = 0; v < L::kVals; ++v) {
            const int ar = WORDS == 2 ? t * 8 + 2 * q + v : t * 16 + 4 * q + v;
            if (ar >= a.rows) continue;
            double tot = red[(((0 * RT + rt) * AT + t) * L::kVals + v) * 64 + lane];
#pragma unroll
            for (int w = 1; w < kWaves; ++w) tot += red[(((w * RT + rt) * AT + t) * L::kVals + v) * 64 + lane];
            const int64_t o = static_cast<int64_t>(ar) * a.ldy + n;
            const double res = a.residual ? static_cast<double>(a.residual[o]) : 0.0;
            a.y[o] = static_cast<float>(tot * post + res);
        }
    }
}

template <int RT, int AT, int WORDS>
hipError_t run(const MmaArgs &a, hipStream_t stream) {
    using L = Layout<RT, AT, WORDS>;
    if (L::kLdsBytes > device_info().lds_per_block) return hipErrorInvalidConfiguration;
    const uint32_t grid = (a.n + a.rows_per_wg - 1) / a.rows_per_wg;
    hipLaunchKernelGGL((mma_kernel<RT, AT, WORDS>), dim3(grid), dim3(kThreads), L::kLdsBytes, stream, a);
    return hipGetLastError();
}

template <int WORDS, int AT>
hipError_t by_rt(int rt, const MmaArgs &a, hipStream_t s) {
    if (rt == 1) return run<1, AT, WORDS>(a, s);
    if (rt == 2) return run<2, AT, WORDS>(a, s);
    if constexpr (AT * WORDS <= 4) return run<4, AT, WORDS>(a, s);
    return hipErrorInvalidValue;
}

// Activation tiles a stack needs, and the widest weight range (in 16-row tiles)
// a workgroup may own with that many tiles.
int act_tiles(int words, int rows) {
    const int per = 16 / words;
    const int t = (rows + per - 1) / per;
    return t <= 1 ? 1 : t <= 2 ? 2 : t <= 4 ? 4 : 8;
}
int max_row_tiles(int words, int at) { return at * words <= 4 ? 4 : 2; }

}  // namespace

bool mma_supports(int mode, int64_t n, int64_t k, int rows, const void *w, const void *hi, const void *lo,
                  const void *scale) {
    if (mode != 1 && mode != 2) return false;
    if (rows < 2 || rows > 64 || k % (kChunkBlocks * kBlock) != 0) return false;
    if (n * (k / kBlock) * kBlockBytes > (int64_t(1) << 30)) return false;
    const auto al16 = [](const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
    if (!al16(w) || !al16(hi) || !al16(scale) || (mode == 2 && !al16(lo))) return false;
    return true;
}

hipError_t launch_mma(int mode, const uint8_t *w, int64_t n, int64_t k, int rows, const int8_t *hi,
                      const int8_t *lo, const float *scale, const float *residual, float *y, int64_t ldy,
                      hipStream_t stream) {
    const int words = mode == 2 ? 2 : 1;
    const int64_t nb = k / kBlock;
    const int at = act_tiles(words, rows);
    const int cus = std::max(1, device_info().cus);
    int64_t per_wg = (n + cus - 1) / cus;
    per_wg = std::min<int64_t>(per_wg, 16 * max_row_tiles(words, at));
    const int rt = per_wg <= 16 ? 1 : per_wg <= 32 ? 2 : 4;
    MmaArgs a;
    a.w = w;
    a.hi = hi;
    a.lo = lo;
    a.scale = scale;
    a.residual = residual;
    a.y = y;
    a.ldy = ldy;
    a.n = static_cast<uint32_t>(n);
    a.k = static_cast<uint32_t>(k);
    a.nb = static_cast<uint32_t>(nb);
    a.row_bytes = static_cast<uint32_t>(nb * kBlockBytes);
    a.w_bytes = static_cast<uint32_t>(n * nb * kBlockBytes);
    a.rows = rows;
    a.rows_per_wg = static_cast<int>(per_wg);
    a.nchunks = static_cast<int>(nb / kChunkBlocks);
    if (words == 2) {
        switch (at) {
            case 1: return by_rt<2, 1>(rt, a, stream);
            case 2: return by_rt<2, 2>(rt, a, stream);
            case 4: return by_rt<2, 4>(rt, a, stream);
            default: return by_rt<2, 8>(rt, a, stream);
        }
    }
    switch (at) {
        case 1: return by_rt<1, 1>(rt, a, stream);
        case 2: return by_rt<1, 2>(rt, a, stream);
        default: return by_rt<1, 4>(rt, a, stream);
    }
}

}  // namespace q8
