// f64mma.hip -- the f32 activation mode (f64 sums) for stacks of 5..64 rows on
// gfx950's f64 matrix cores, every weight block read once for the whole stack
// (codegen_cuda::lane page, description: the f32 activation numerics and a
// stack's single pass over each weight; model::author page, Functions: prefill,
// decode_batch).
//
// v_mfma_f64_16x16x4f64 multiplies a 16 x 4 operand A by a 4 x 16 operand B.
// Here A is 16 activation rows and B 16 weight rows: lane l supplies row l % 16
// at column l / 16 of either, and gets back the results of activation rows
// l / 16 + 4 v (v = 0..3) against weight row l % 16.  A block's 32 columns are
// dealt so that lane l's column at step s is 8 (l / 16) + s: every lane needs 8
// consecutive quants of its weight row and 8 consecutive f32 values of its
// activation row.  int8 and f32 values are exact in f64 and so are their
// products (at most 32 significant bits), so each block's p = sum_j q_j x_j is
// summed in f64 by 8 chained MFMAs, and d * p joins the output's f64
// accumulator with one fused multiply-add: the block sum, then the scale, as
// the numerics define the f32 mode.  Each output is rounded to f32 once, after
// the residual is added in f64.
//
// Work split: one workgroup per one or two 16-row weight tiles.  Its 8 waves
// take the blocks of k in turn (wave g: blocks g, g + 8, ...) for every weight
// and activation tile, so each weight block is read by one wave of one
// workgroup; the waves' partial sums are added in wave order at the end.
// Operands come from memory with range-checked buffer loads, a chunk of D
// blocks ahead of the MFMAs.  Every workgroup reads the stack (through L2); HBM
// serves each weight block one time.  With a caller workspace (the K split,
// f64_mma_split_kernel) a workgroup takes two tiles and a 2nd, 4th or 8th of
// k, and the parts of a tile pair are added across workgroups at the end.
#include <algorithm>

#include "device.h"
#include "launch.h"

namespace q8 {
namespace {

constexpr int kWaves = 8;                 // K groups per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr uint32_t kBufferDword3 = 0x00020000u;
constexpr int64_t kMaxWeightBytes = int64_t(1) << 30;  // one launch's weights
constexpr int64_t kMaxK = int64_t(1) << 22;           // keeps 65 rows of x under 2^31 bytes
// Below 5 rows the f64 GEMV is faster (4 rows of 4096 x 4096: 14 us against
// about 16 us here); from 5 rows on it falls far behind (43 us at 6 rows).
constexpr int kMinRows = 5;
constexpr int kSplitMinBlocks = 16;  // blocks per workgroup of a split: two per wave

typedef double v4d __attribute__((ext_vector_type(4)));
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

struct F64Args {
    const uint8_t *w;        // Q8_0 blocks [n][nb] of this launch's rows
    const float *x;          // [rows][k]
    const float *residual;   // [rows][ldy] or null
    float *y;                // [rows][ldy]
    int64_t ldy;
    uint32_t n;              // weight rows of this launch
    uint32_t k;
    uint32_t nb;
    uint32_t w_bytes;        // n * nb * 34
    int rows;                // activation rows (5..64)
    // K split over workgroups (f64_mma_split_kernel): workgroup g takes weight
    // tile range g / ksplit and blocks [nb / ksplit * (g % ksplit), + nb / ksplit);
    // the ranges' partial totals meet in a caller workspace.
    int ksplit;
    double *ks_part;         // [ranges][ksplit][RT * AT * 4 * 64] f64 partials
    uint32_t *ks_count;      // [ranges] arrivals, zero between calls
};

// One block's operands for this lane: for each of its RT weight rows the
// dword-aligned 12 bytes holding its 8 quants, and 8 f32 activation values per
// activation tile.  The block's binary16 scale is not loaded on its own: the
// window of a row's first lane (lane / 16 == 0) starts at the block or 2 bytes
// before it, so its first dword holds the scale, which math_block passes to the
// row's other lanes.
template <int RT, int AT>
struct Ops {
    u32x3 win[RT];
    f32x4 x[AT][2];
};

// Block b of weight rows row + 16 rt for this lane (`live` false: every load
// reads zeros).  The lane's quants start at byte 2 + 8 (lane / 16) of the
// block; the 12 bytes from the dword at or before them never reach past the
// matrix, since k is a multiple of 64 and the last block of a row starts 2
// bytes past a dword boundary.
template <int RT, int AT>
__device__ __forceinline__ void load_ops(const F64Args &a, __amdgpu_buffer_rsrc_t rw, __amdgpu_buffer_rsrc_t rx,
                                         uint32_t row, uint32_t b, int lane, bool live, Ops<RT, AT> &o) {
    const uint32_t kq = static_cast<uint32_t>(lane >> 4), r16 = static_cast<uint32_t>(lane & 15);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const uint32_t wrow = row + 16 * rt;
        const uint32_t blk = wrow * a.nb + b;
        const uint32_t dead = oob_bit(live && wrow < a.n);
        o.win[rt] = __builtin_amdgcn_raw_buffer_load_b96(rw, ((blk * kBlockBytes + 8 * kq) & ~3u) | dead, 0, 0);
    }
    const uint32_t x0 = (r16 * a.k + b * kBlock + 8 * kq) * 4;  // tile t adds 64 t k bytes
#pragma unroll
    for (int t = 0; t < AT; ++t) {
        const uint32_t r = static_cast<uint32_t>(t * 16) + r16;
        const uint32_t off = (x0 + static_cast<uint32_t>(t) * 64u * a.k) | oob_bit(live && r < static_cast<uint32_t>(a.rows));
        o.x[t][0] = __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, 0);
        o.x[t][1] = __builtin_amdgcn_raw_buffer_load_b128(rx, off + 16, 0, 0);
    }
}

// d * (sum of the block's 32 products) into acc, for every weight and
// activation tile.  Block b's parity decides where its quants sit in a window
// (the window starts at the block when b is even, 2 bytes before it when odd),
// and where the scale sits in the first dword of the row's first lane, which
// every lane of the row reads with ds_bpermute (lane_row4 = 4 (lane % 16)).
// Each activation value is converted once and used for every weight tile.
template <int RT, int AT>
__device__ __forceinline__ void math_block(const Ops<RT, AT> &o, uint32_t b, int lane_row4, v4d (&acc)[RT][AT]) {
    const uint32_t sel = window_selector(b);
    double q[RT][8];
    double d[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const uint32_t lo = __builtin_amdgcn_perm(o.win[rt].y, o.win[rt].x, sel);
        const uint32_t hi = __builtin_amdgcn_perm(o.win[rt].z, o.win[rt].y, sel);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            q[rt][s] = static_cast<double>(static_cast<int8_t>(lo >> (8 * s)));
            q[rt][4 + s] = static_cast<double>(static_cast<int8_t>(hi >> (8 * s)));
        }
        const uint32_t own = (b & 1) ? (o.win[rt].x >> 16) : (o.win[rt].x & 0xffffu);
        const uint32_t dbits = static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(lane_row4, static_cast<int>(own)));
        d[rt] = static_cast<double>(f16_bits_to_float(dbits));
    }
#pragma unroll
    for (int t = 0; t < AT; ++t) {
        const float xs[8] = {o.x[t][0].x, o.x[t][0].y, o.x[t][0].z, o.x[t][0].w,
                             o.x[t][1].x, o.x[t][1].y, o.x[t][1].z, o.x[t][1].w};
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            v4d p = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
            for (int s = 0; s < 8; ++s)
                p = __builtin_amdgcn_mfma_f64_16x16x4f64(static_cast<double>(xs[s]), q[rt][s], p, 0, 0, 0);
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[rt][t][v] = __builtin_fma(d[rt], p[v], acc[rt][t][v]);
        }
    }
}

// LDS of the waves' partial sums: 112 KiB at two weight and four activation tiles.
constexpr size_t park_bytes(int rt, int at) { return size_t(kWaves - 1) * rt * at * 4 * 64 * sizeof(double); }

// The last workgroup of a split range, wave 0: total f (= (rt AT + t) 4 + v)
// of this lane = sum over parts s (in order) of parts[s * kTot + 64 f + lane],
// into acc[rt][t][v].  The loads of a group of totals, all KS parts of each (at
// most 32 loads), are issued at once: one memory round trip per group.
template <int KS, int RT, int AT>
__device__ __forceinline__ void combine_parts(const double *parts, int lane, v4d (&acc)[RT][AT]) {
    constexpr int NV = RT * AT * 4;
    constexpr int kTot = NV * 64;
    constexpr int G = 32 / KS < NV ? 32 / KS : NV;
#pragma unroll
    for (int f0 = 0; f0 < NV; f0 += G) {
        double p[G][KS];
#pragma unroll
        for (int g = 0; g < G; ++g)
            if (f0 + g < NV) {
#pragma unroll
                for (int s = 0; s < KS; ++s)
                    p[g][s] = __hip_atomic_load(parts + static_cast<size_t>(s) * kTot + (f0 + g) * 64 + lane,
                                                __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
#pragma unroll
        for (int g = 0; g < G; ++g)
            if (f0 + g < NV) {
                double t = p[g][0];
#pragma unroll
                for (int s = 1; s < KS; ++s) t += p[g][s];
                const int f = f0 + g;
                acc[f / (AT * 4)][(f / 4) % AT][f % 4] = t;
            }
    }
}

// RT 16-row weight tiles per workgroup (each wave covers all of them),
// AT 16-row activation tiles.  SPLIT: this workgroup takes 1/ksplit of K for
// its tiles, and the last of a range's workgroups to finish adds the partial
// totals (launched as f64_mma_split_kernel, so that f64_mma_kernel carries none
// of it).
template <int RT, int AT, bool SPLIT>
__device__ __forceinline__ void f64_body(const F64Args &a) {
    constexpr int D = 8 / (RT * AT);  // blocks per chunk: 64 MFMAs of work between a chunk's loads and its use
    __shared__ double park[kWaves - 1][RT][AT][4][64];
    static_assert(sizeof(park) == park_bytes(RT, AT));
    const int lane = threadIdx.x & 63;
    const int lane_row4 = (lane & 15) << 2;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int ksplit = SPLIT ? a.ksplit : 1;
    const uint32_t range = blockIdx.x / static_cast<uint32_t>(ksplit);
    const uint32_t split = blockIdx.x - range * static_cast<uint32_t>(ksplit);
    const uint32_t row = range * (16u * RT) + static_cast<uint32_t>(lane & 15);
    const __amdgpu_buffer_rsrc_t rw =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(a.w), 0, a.w_bytes, kBufferDword3);
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float *>(a.x), 0, static_cast<uint32_t>(a.rows) * a.k * 4, kBufferDword3);

    v4d acc[RT][AT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int t = 0; t < AT; ++t) acc[rt][t] = v4d{0.0, 0.0, 0.0, 0.0};

    // this wave's blocks: wave + kWaves j for j < mine, in chunks of D blocks
    // loaded into two register buffers in turn, each chunk's loads issued
    // before the previous chunk's MFMAs (the scheduler barriers keep that
    // order).  The loop runs while a whole pair of chunks and one more block
    // remain, so every refill it issues reads at least one live block; the
    // last one or two chunks are finished after it without refills.  Blocks
    // past the wave's last read zeros and add exact zeros.
    const int nb = static_cast<int>(a.nb) / ksplit;  // this workgroup's blocks: kb0 .. kb0 + nb - 1
    const uint32_t kb0 = split * static_cast<uint32_t>(nb);
    const int mine = wave < nb ? (nb - wave + kWaves - 1) / kWaves : 0;
    const int last = std::max(mine - 1, 0);
    auto block_of = [&](int j) { return kb0 + static_cast<uint32_t>(wave + kWaves * std::min(j, last)); };
    Ops<RT, AT> ping[D], pong[D];
#pragma unroll
    for (int c = 0; c < D; ++c) load_ops<RT, AT>(a, rw, rx, row, block_of(c), lane, c < mine, ping[c]);
    int j0 = 0;
    for (; j0 + 2 * D < mine; j0 += 2 * D) {
#pragma unroll
        for (int c = 0; c < D; ++c)
            load_ops<RT, AT>(a, rw, rx, row, block_of(j0 + D + c), lane, j0 + D + c < mine, pong[c]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int c = 0; c < D; ++c) math_block<RT, AT>(ping[c], block_of(j0 + c), lane_row4, acc);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int c = 0; c < D; ++c)
            load_ops<RT, AT>(a, rw, rx, row, block_of(j0 + 2 * D + c), lane, j0 + 2 * D + c < mine, ping[c]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int c = 0; c < D; ++c) math_block<RT, AT>(pong[c], block_of(j0 + D + c), lane_row4, acc);
        __builtin_amdgcn_sched_barrier(0);
    }
    if (j0 + D < mine) {  // two chunks left: chunk j0 is in ping
#pragma unroll
        for (int c = 0; c < D; ++c)
            load_ops<RT, AT>(a, rw, rx, row, block_of(j0 + D + c), lane, j0 + D + c < mine, pong[c]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int c = 0; c < D; ++c) math_block<RT, AT>(ping[c], block_of(j0 + c), lane_row4, acc);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int c = 0; c < D; ++c) math_block<RT, AT>(pong[c], block_of(j0 + D + c), lane_row4, acc);
    } else if (j0 < mine) {  // one chunk left
#pragma unroll
        for (int c = 0; c < D; ++c) math_block<RT, AT>(ping[c], block_of(j0 + c), lane_row4, acc);
    }

    // partial sums of waves 1..7 through LDS, added to wave 0's in wave order
    if (wave > 0) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int t = 0; t < AT; ++t)
#pragma unroll
                for (int v = 0; v < 4; ++v) park[wave - 1][rt][t][v][lane] = acc[rt][t][v];
    }
    __syncthreads();
    if constexpr (!SPLIT) {
        if (wave != 0 || row >= a.n) return;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const uint32_t wrow = row + 16 * rt;
            if (rt > 0 && wrow >= a.n) continue;
#pragma unroll
            for (int t = 0; t < AT; ++t)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    double tot = acc[rt][t][v];
#pragma unroll
                    for (int w = 0; w < kWaves - 1; ++w) tot += park[w][rt][t][v][lane];
                    const int r = t * 16 + (lane >> 4) + 4 * v;
                    if (r >= a.rows) continue;
                    const int64_t o = static_cast<int64_t>(r) * a.ldy + wrow;
                    const double res = a.residual ? static_cast<double>(a.residual[o]) : 0.0;
                    a.y[o] = static_cast<float>(tot + res);
                }
        }
        return;
    }
    if (wave != 0) return;
    // wave 0's totals, in wave order (as the unsplit kernel adds them), in place
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int t = 0; t < AT; ++t)
#pragma unroll
            for (int v = 0; v < 4; ++v)
#pragma unroll
                for (int w = 0; w < kWaves - 1; ++w) acc[rt][t][v] += park[w][rt][t][v][lane];
    {
        // K split: these totals are one of ksplit parts of the range's.  Wave 0 writes
        // them to the workspace as agent-scope atomic stores (through the XCD's
        // L2 to the device-coherent level) and waits for them; lane 0 then
        // counts the workgroup in.  The last to count reads every part back
        // (its own included) and adds them in part order: the same bits
        // whichever workgroup is last.
        constexpr int kTot = RT * AT * 4 * 64;
        double *parts = a.ks_part + static_cast<size_t>(range) * ksplit * kTot;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int t = 0; t < AT; ++t)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    __hip_atomic_store(parts + static_cast<size_t>(split) * kTot + ((rt * AT + t) * 4 + v) * 64 + lane,
                                       acc[rt][t][v], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        uint32_t done = 0;
        if (lane == 0) done = __hip_atomic_fetch_add(a.ks_count + range, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        done = __builtin_amdgcn_readfirstlane(done);
        if (done != static_cast<uint32_t>(ksplit - 1)) return;
        if (ksplit == 2)
            combine_parts<2, RT, AT>(parts, lane, acc);
        else if (ksplit == 4)
            combine_parts<4, RT, AT>(parts, lane, acc);
        else
            combine_parts<8, RT, AT>(parts, lane, acc);
        if (lane == 0) __hip_atomic_store(a.ks_count + range, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (row >= a.n) return;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const uint32_t wrow = row + 16 * rt;
        if (rt > 0 && wrow >= a.n) continue;
#pragma unroll
        for (int t = 0; t < AT; ++t)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int r = t * 16 + (lane >> 4) + 4 * v;
                if (r >= a.rows) continue;
                const int64_t o = static_cast<int64_t>(r) * a.ldy + wrow;
                const double res = a.residual ? static_cast<double>(a.residual[o]) : 0.0;
                a.y[o] = static_cast<float>(acc[rt][t][v] + res);
            }
    }
}

template <int RT, int AT>
__global__ __launch_bounds__(kThreads) void f64_mma_kernel(F64Args a) {
    f64_body<RT, AT, false>(a);
}

template <int RT, int AT>
__global__ __launch_bounds__(kThreads) void f64_mma_split_kernel(F64Args a) {
    f64_body<RT, AT, true>(a);
}

template <int RT, int AT>
hipError_t run(const F64Args &a, hipStream_t stream) {
    constexpr int64_t kTile = 16 * RT;
    const int64_t row_bytes = static_cast<int64_t>(a.nb) * kBlockBytes;
    const int64_t slice = std::max<int64_t>(kTile, (kMaxWeightBytes / row_bytes) / kTile * kTile);
    const int64_t n = a.n;
    for (int64_t r0 = 0; r0 < n; r0 += slice) {
        F64Args s = a;
        s.w = a.w + r0 * row_bytes;
        s.n = static_cast<uint32_t>(std::min(slice, n - r0));
        s.w_bytes = static_cast<uint32_t>(s.n * row_bytes);
        s.y = a.y + r0;
        s.residual = a.residual ? a.residual + r0 : nullptr;
        const unsigned grid = static_cast<unsigned>((s.n + kTile - 1) / kTile);
        f64_mma_kernel<RT, AT><<<grid, kThreads, 0, stream>>>(s);
        if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    }
    return hipSuccess;
}

// K split: two 16-row weight tiles a workgroup (each activation load and
// conversion feeding two MFMA chains, as on tall matrices) over a range's
// ksplit parts of K, for matrices where the unsplit launch keeps one tile a
// workgroup (at most 16 rows per CU).  Measured (graphs of 20 launches,
// unsplit against split): 4096 x 14336 16 rows 55.0 against 47.4 us, 64 rows
// 139.8 against 126.2; 2048 x 14336 64 rows 139.4 against 69.5 (the unsplit
// launch fills half the CUs); 1024 x 14336 64 rows 138.1 against 43.6; 4096 x
// 4096 64 rows 46.3 against 43.8.  Not taken for one activation tile on a
// full chip with under 128 blocks a part: 4096 x 4096 at 6-12 rows measured
// 16.5-17.4 against 17.1-17.5 us.
struct F64Split {
    int at = 0;
    int ksplit = 1;          // 1: no split
    int64_t ranges = 0;
    int64_t bytes = 0;
};

F64Split f64_split_plan(int64_t n, int64_t k, int rows) {
    F64Split p;
    const DeviceInfo dev = device_info();
    const int64_t cus = std::max(1, dev.cus);
    if (rows < kMinRows || rows > 64 || n < 1 || k < 64 || k % 64 != 0 || k > kMaxK) return p;
    if (n > 16 * cus || n * (k / kBlock) * kBlockBytes > kMaxWeightBytes) return p;
    const int at = rows <= 16 ? 1 : rows <= 32 ? 2 : 4;
    if (park_bytes(2, at) > static_cast<size_t>(dev.lds_per_block)) return p;
    const int64_t nb = k / kBlock;
    const int64_t ranges = (n + 31) / 32;
    int split = 1;
    for (int c : {8, 4, 2})
        if (ranges * c <= cus && nb % c == 0 && nb / c >= kSplitMinBlocks) {
            split = c;
            break;
        }
    if (split == 1) return p;
    if (at == 1 && n > 8 * cus && nb / split < 128) return p;
    p.at = at;
    p.ksplit = split;
    p.ranges = ranges;
    p.bytes = split_count_bytes(static_cast<int>(cus)) + ranges * split * (2 * at * 4 * 64) * 8;
    return p;
}

template <int AT>
hipError_t run_split(const F64Args &a, hipStream_t stream) {
    const unsigned grid = static_cast<unsigned>((a.n + 31) / 32 * a.ksplit);
    f64_mma_split_kernel<2, AT><<<grid, kThreads, 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace

bool f64_mma_supports(int64_t n, int64_t k, int rows, const void *x) {
    return rows >= kMinRows && rows <= 64 && n >= 1 && k >= 64 && k % 64 == 0 && k <= kMaxK &&
           (reinterpret_cast<uintptr_t>(x) & 15) == 0;
}

hipError_t launch_f64_mma(const uint8_t *w, int64_t n, int64_t k, int rows, const float *x, const float *residual,
                          float *y, int64_t ldy, hipStream_t stream) {
    F64Args a;
    a.w = w;
    a.x = x;
    a.residual = residual;
    a.y = y;
    a.ldy = ldy;
    a.n = static_cast<uint32_t>(n);  // per-launch slices are at most 2^30 bytes of rows
    a.k = static_cast<uint32_t>(k);
    a.nb = static_cast<uint32_t>(k / kBlock);
    a.w_bytes = 0;
    a.rows = rows;
    a.ksplit = 1;
    a.ks_part = nullptr;
    a.ks_count = nullptr;
    // Two weight tiles a workgroup where that takes fewer rounds of
    // workgroups over the CUs, at about 1.65 times the time of a one-tile
    // round: each activation load and conversion then feeds two MFMA chains.
    const DeviceInfo dev = device_info();
    const int64_t cus = std::max(1, dev.cus);
    const int64_t rounds1 = (a.n + 16 * cus - 1) / (16 * cus), rounds2 = (a.n + 32 * cus - 1) / (32 * cus);
    const bool two = 5 * rounds2 < 3 * rounds1;
    if (rows <= 16) return two ? run<2, 1>(a, stream) : run<1, 1>(a, stream);
    if (rows <= 32) return two ? run<2, 2>(a, stream) : run<1, 2>(a, stream);
    if (two && park_bytes(2, 4) <= static_cast<size_t>(dev.lds_per_block)) return run<2, 4>(a, stream);
    return run<1, 4>(a, stream);
}

int64_t f64_ksplit_bytes(int64_t n, int64_t k, int rows) {
    const F64Split p = f64_split_plan(n, k, rows);
    return p.ksplit > 1 ? p.bytes : 0;
}

hipError_t launch_f64_mma_ksplit(const uint8_t *w, int64_t n, int64_t k, int rows, const float *x,
                                 const float *residual, float *y, void *workspace, hipStream_t stream) {
    const F64Split p = f64_split_plan(n, k, rows);
    if (p.ksplit <= 1 || !workspace) return hipErrorInvalidValue;
    F64Args a;
    a.w = w;
    a.x = x;
    a.residual = residual;
    a.y = y;
    a.ldy = n;
    a.n = static_cast<uint32_t>(n);
    a.k = static_cast<uint32_t>(k);
    a.nb = static_cast<uint32_t>(k / kBlock);
    a.w_bytes = static_cast<uint32_t>(n * (k / kBlock) * kBlockBytes);
    a.rows = rows;
    a.ksplit = p.ksplit;
    a.ks_count = static_cast<uint32_t *>(workspace);
    a.ks_part = reinterpret_cast<double *>(static_cast<uint8_t *>(workspace) +
                                           split_count_bytes(std::max(1, device_info().cus)));
    if (p.at == 1) return run_split<1>(a, stream);
    if (p.at == 2) return run_split<2>(a, stream);
    return run_split<4>(a, stream);
}

}  // namespace q8
