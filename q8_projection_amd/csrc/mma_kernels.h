// mma_kernels.h -- the projection for stacks of 2..64 activation rows on
// gfx950's int8 matrix cores, with every operand staged through an LDS ring.
// Kernel templates and their launch logic; mma.hip instantiates the projection
// and mma_sums.hip the block-sum export (SUMS: the same kernel writes each
// block's exact int32 MFMA results, S_hi and S_lo, to a caller buffer; the
// scales are then not read).
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
// no VGPR holds staged data.  The W waves of the workgroup issue the copies
// together (each lane's offsets are computed once; a chunk adds a constant) and
// split the chunk's blocks for the math; one barrier per chunk hands a ring
// slot from the copies to the MFMAs, and the copies run kDepth - 1 chunks ahead.
//
// Math.  v_mfma_i32_16x16x32_i8 takes one block per instruction: operand A is
// 16 activation columns, operand B 16 weight rows, both 32 int8 along K, and the
// result is their 16x16 exact int32 block sums.  Lane l supplies column (or
// row) l%16, bytes 8(l/16)..8(l/16)+7 of the block, and receives columns
// 4(l/16)..4(l/16)+3 of weight row l%16.  In the two-word mode the 16 columns of
// a tile are the hi and lo words of 8 activation rows, ordered so that each lane
// receives both words of two rows: T = 128 S_hi + S_lo is formed exactly in
// int32.  Every block term (d * s) * T is accumulated in f64; at the end the
// waves' partials are added pairwise in a fixed tree order and each output is
// rounded once to f32.
//
// The copies are issued with inline assembly on purpose: the compiler cannot
// tell ring slots apart and would otherwise wait for every outstanding copy
// before each LDS read.  The waits on the copies are explicit (vmcnt) and the
// barrier carries release/acquire fences for the LDS reads.
#pragma once

#include <algorithm>

#include "device.h"
#include "launch.h"

namespace q8 {
namespace {

#pragma clang fp contract(off)

constexpr int kChunkBlocks = 8;                            // blocks per chunk
constexpr int kRowChunk = kChunkBlocks * kBlockBytes;      // 272 bytes of one weight row
constexpr int kRowGranules = kRowChunk / 16;               // 17
constexpr int kActChunk = kChunkBlocks * kBlock;           // 256 activation bytes per row and word
constexpr int kTileBytes = 16 * kActChunk;                 // one 16-column activation tile
constexpr int kCopyBytes = 1024;                           // one copy instruction: 64 lanes x 16 B
constexpr int kColGranules = kActChunk / 16;               // 16-byte granules of one column's chunk
constexpr int kColsPerCopy = kCopyBytes / kActChunk;       // column slots one copy fills
constexpr int kTileCopies = kTileBytes / kCopyBytes;       // copies of one tile
static_assert(kChunkBlocks % 8 == 0 && kActChunk <= kCopyBytes, "a chunk is 8, 16 or 32 blocks");
constexpr int kRingBudget = 156 * 1024;  // LDS for the ring (gfx950: 160 KB per workgroup)
constexpr int kMaxDepth = 12;
constexpr int kInFlight = 44 * 1024;  // copy bytes kept in flight per workgroup (measured best)
constexpr uint32_t kBufferDword3 = 0x00020000u;
constexpr uint32_t kOob = 0x80000000u;
constexpr int kWaveMaxRt = 1;     // single-tile stacks on matrices this short use the wave-private kernel
constexpr int kWaveWaves = 8;
constexpr int kWaveDepth = 2;
constexpr int64_t kMaxMmaWeightBytes = int64_t(1) << 30;  // one launch's weights (buffer offsets < 2^31)

typedef int v4i __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) uint8_t *lds_ptr_t;

// Sizes of one ring slot and of the ring, per instantiation.
//   RT: 16-row weight tiles per workgroup; TT: 16-column activation tiles;
//   GR x GA x GB waves: wave w takes the activation tiles of group w % GA, the
//   weight tiles of group (w / GA) % GR and the blocks of group w / (GA GR) of
//   every chunk.  Block groups (GB > 1) split K, and their partial sums are
//   added by a tree at the end; weight and activation groups split the outputs.
template <int RT, int TT, int WORDS, int GR, int GA, int GB>
struct Layout {
    static constexpr int W = GR * GA * GB;                     // waves per workgroup
    static constexpr int kAT = TT / GA;                        // activation tiles per wave
    static constexpr int kRTW = RT / GR;                       // weight tiles per wave
    static constexpr int kRows = RT * 16;                      // weight rows a workgroup may own
    static constexpr int kActRows = TT * 16 / WORDS;           // activation rows the tiles hold
    static constexpr int kWCopies = (kRows * kRowGranules + 63) / 64;
    static constexpr int kACopies = TT * kTileCopies;          // 16 columns x kActChunk bytes per tile
    static constexpr int kSCopies = kActRows * kChunkBlocks / 64;  // 4-byte copies of the scales, [block][row]
    static constexpr int kCopies = kWCopies + kACopies + kSCopies;
    static constexpr int kPerWave = (kCopies + W - 1) / W;     // copies of the first kCopies % W waves
    static constexpr int kPerWaveLow = kCopies / W;            // copies of the others
    static constexpr int kSlotBytes = (kWCopies + kACopies) * kCopyBytes + kSCopies * 256;
    static constexpr int kAOff = kWCopies * kCopyBytes;
    static constexpr int kSOff = kAOff + kACopies * kCopyBytes;
    // enough slots for about kInFlight bytes of copies ahead of the math (deeper
    // rings measured slower), at least three, within the LDS budget
    static constexpr int kDepth =
        std::max(3, std::min({kMaxDepth, kRingBudget / kSlotBytes, 1 + kInFlight / kSlotBytes}));
    static constexpr int kBlocksPerWave = kChunkBlocks / GB;
    static constexpr int kVals = WORDS == 2 ? 2 : 4;           // f64 accumulators per lane and tile pair
    static constexpr int kAccBytes = kRTW * kAT * kVals * 64 * 8; // one wave's accumulators
    static constexpr int kLdsBytes = std::max(kDepth * kSlotBytes, (W / 2) * kAccBytes);
    static_assert(TT % GA == 0 && RT % GR == 0 && kChunkBlocks % GB == 0 && (GB & (GB - 1)) == 0, "wave split");
    static_assert(W <= 16, "at most 1024 threads");
    static_assert(kRingBudget / kSlotBytes >= 3, "the ring needs at least three slots");
    // a wave never has more vector-memory operations in flight than vmcnt can
    // count (six bits)
    static_assert(kPerWave * (kDepth - 1) <= 63, "outstanding copies exceed the vmcnt range");
    static_assert(RT * TT * kVals * 64 * 8 <= kLdsBytes, "room for the totals");
    static_assert(kActRows * kChunkBlocks % 64 == 0, "whole scale copies");
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
    uint32_t lo_oob;         // kOob for a one-word stack run in the two-word layout, else 0
    int32_t *sums;           // block-sum export [rows][sums_ld][nb][sums_words], or null
    int64_t sums_ld;         // weight rows of the whole call (the export's row stride)
    int sums_words;          // 2 for a two-word stack, else 1
    // K split over workgroups (ksplit > 1): workgroup g takes row range
    // g / ksplit and chunks [nchunks * (g % ksplit), + nchunks); the ranges'
    // partial sums meet in a caller workspace (ks_part, ks_count: below).
    int ksplit;
    double *ks_part;         // [ranges][ksplit][RT * TT * kVals * 64] f64 partials
    uint32_t *ks_count;      // [ranges] arrivals, zero between calls
};

struct Rsrcs {
    __amdgpu_buffer_rsrc_t w, hi, lo, s;
    uint32_t lo_oob;  // kOob: the lo words read as zeros (a one-word stack in the two-word layout)
};

// One direct-to-LDS copy: lane i's 16 bytes at buffer offset `off` land at LDS
// address lds + 16 i (copy4: 4 bytes at lds + 4 i).  An offset with bit 31 set
// reads zeros and touches no memory.
__device__ __forceinline__ void copy16(__amdgpu_buffer_rsrc_t r, uint32_t lds, uint32_t off) {
    asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(off), "s"(r), "{m0}"(lds) : "memory");
}
__device__ __forceinline__ void copy4(__amdgpu_buffer_rsrc_t r, uint32_t lds, uint32_t off) {
    asm volatile("buffer_load_dword %0, %1, 0 offen lds" ::"v"(off), "s"(r), "{m0}"(lds) : "memory");
}

template <int N>
__device__ __forceinline__ void wait_copies() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Hand LDS over between waves: this wave's LDS accesses are complete (release)
// and the other waves' (including copies already waited for with vmcnt) are
// visible (acquire).
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

// What copy i of a chunk reads.  Layout of a slot:
//   [0, kAOff)      weight rows, row-major, 272 bytes each (17 granules)
//   [kAOff, kSOff)  activation tiles: 16 column slots x 256 bytes, the 16-byte
//                   granules of slot s XOR-permuted by s
//   [kSOff, ...)    activation scales, [block][row] f32 (copied 4 bytes a lane,
//                   so that a lane's 4 or 2 rows of one block are adjacent)
// The result is this lane's offset for chunk 0 (bit 31 set where the lane reads
// nothing); chunk c adds c * kRowChunk, c * kActChunk or c * kChunkBlocks * 4 to it.
template <int RT, int TT, int WORDS, int GR, int GA, int GB>
__device__ __forceinline__ uint32_t plan_copy(const MmaArgs &a, int i, int lane, uint32_t r0, int rcount) {
    using L = Layout<RT, TT, WORDS, GR, GA, GB>;
    if (i < L::kWCopies) {
        const int g = i * 64 + lane;
        const int row = g / kRowGranules;
        const int part = g - row * kRowGranules;
        return ((r0 + row) * a.row_bytes + 16 * part) | oob_bit(row < rcount);
    }
    if (i < L::kWCopies + L::kACopies) {
        const int ia = i - L::kWCopies;
        const int t = ia / kTileCopies;
        const int s = (ia % kTileCopies) * kColsPerCopy + lane / kColGranules;  // column slot
        const int g = (lane % kColGranules) ^ s;  // granule of the row's chunk bytes
        const int row = WORDS == 2 ? t * 8 + (s & 7) : t * 16 + s;
        return (static_cast<uint32_t>(row) * a.k + 16 * g) | oob_bit(row < a.rows);
    }
    if (i < L::kCopies) {
        const int f = (i - L::kWCopies - L::kACopies) * 64 + lane;  // [block][row] position
        const int j = f / L::kActRows, row = f % L::kActRows;
        return (static_cast<uint32_t>(row) * a.nb * 4 + 4 * j) | oob_bit(row < a.rows);
    }
    return kOob;
}

// Copies of chunk kc0 + c into the slot at LDS address `slot` (chunk c of the
// workgroup's K range; c >= nchunks reads nothing): copy i is issued by
// wave i % W, so a wave issues kPerWave or kPerWaveLow copies per chunk, the
// same number for every chunk (chunks past the end read nothing), and its
// vmcnt waits are exact.
template <int RT, int TT, int WORDS, int GR, int GA, int GB>
__device__ __forceinline__ void issue_chunk(const Rsrcs &rs,
                                            const uint32_t (&base)[Layout<RT, TT, WORDS, GR, GA, GB>::kPerWave],
                                            uint32_t slot, int c, int nchunks, int wave, int kc0) {
    using L = Layout<RT, TT, WORDS, GR, GA, GB>;
    constexpr int W = L::W;
    const uint32_t chunk_oob = c < nchunks ? 0u : kOob;
#pragma unroll
    for (int u = 0; u < L::kPerWave; ++u) {
        const int i = wave + W * u;  // wave-uniform copy index
        if (i >= L::kCopies) {
            // not this wave's: the copies are dealt round-robin
        } else if (i < L::kWCopies) {
            copy16(rs.w, slot + i * kCopyBytes, (base[u] + (kc0 + c) * kRowChunk) | chunk_oob);
        } else if (i < L::kWCopies + L::kACopies) {
            // slots 0..7 hold hi rows, 8..15 lo rows; a copy fills kColsPerCopy of them
            const bool lo = WORDS == 2 && ((i - L::kWCopies) % kTileCopies) * kColsPerCopy >= 8;
            copy16(lo ? rs.lo : rs.hi, slot + i * kCopyBytes,
                   (base[u] + (kc0 + c) * kActChunk) | chunk_oob | (lo ? rs.lo_oob : 0u));
        } else {
            copy4(rs.s, slot + L::kSOff + (i - L::kWCopies - L::kACopies) * 256,
                  (base[u] + (kc0 + c) * (kChunkBlocks * 4)) | chunk_oob);
        }
    }
}

// Lane-constant LDS offsets (relative to a slot) of one block's operands.
struct BlockOffsets {
    int j;         // the block's index within the chunk
    uint32_t a;    // activation operand of the wave's first tile (its tile t: + t * kTileBytes)
    uint32_t b;    // dword-aligned start of the weight operand of the wave's first row tile (+ rt * 16 * 272)
    uint32_t d;    // the weight row's block scale (+ rt * 16 * 272)
    uint32_t s;    // activation scales of the lane's result columns (4 or 2 adjacent), the wave's first tile
    uint32_t sel;  // v_perm selector realigning the weight operand (uniform)
};

template <int RT, int TT, int WORDS, int GR, int GA, int GB>
__device__ __forceinline__ BlockOffsets block_offsets(int j, int t0, int r0t, int lane) {
    using L = Layout<RT, TT, WORDS, GR, GA, GB>;
    const int q = lane >> 4, c16 = lane & 15;
    const int as = act_slot<WORDS>(c16);
    const int boff = j * kBlockBytes + 2 + 8 * q;  // first quant byte of the lane's weight operand
    BlockOffsets o;
    o.j = j;
    o.a = L::kAOff + t0 * kTileBytes + as * kActChunk + ((((j << 1) + (q >> 1)) ^ as) << 4) + ((q & 1) << 3);
    o.b = (r0t * 16 + c16) * kRowChunk + (boff & ~3);
    o.d = (r0t * 16 + c16) * kRowChunk + j * kBlockBytes;
    o.s = L::kSOff + (j * L::kActRows + t0 * (16 / WORDS) + (WORDS == 2 ? 2 * q : 4 * q)) * 4;
    o.sel = (boff & 2) ? 0x05040302u : 0x03020100u;
    return o;
}

// One block's operands for this wave, read from the slot: the activation
// operands and scales of its tiles, the weight window and scale of each of its
// row tiles.  Every LDS read of a block (or of several) is issued before any
// of them is used, so their latencies overlap.
template <int RT, int TT, int WORDS, int GR, int GA, int GB>
struct BlockOps {
    using L = Layout<RT, TT, WORDS, GR, GA, GB>;
    long a[L::kAT];
    float s[L::kAT][L::kVals];
    uint32_t w[L::kRTW][3];
    uint16_t d[L::kRTW];
};

template <int RT, int TT, int WORDS, int GR, int GA, int GB>
__device__ __forceinline__ void load_block(const uint8_t *slot, const BlockOffsets &o,
                                           BlockOps<RT, TT, WORDS, GR, GA, GB> &op) {
    using L = Layout<RT, TT, WORDS, GR, GA, GB>;
#pragma unroll
    for (int t = 0; t < L::kAT; ++t) {
        op.a[t] = *reinterpret_cast<const long *>(slot + o.a + t * kTileBytes);
        const float *ps = reinterpret_cast<const float *>(slot + o.s + t * (16 / WORDS) * 4);
        if constexpr (WORDS == 2) {
            const float2 sv = *reinterpret_cast<const float2 *>(ps);
            op.s[t][0] = sv.x;
            op.s[t][1] = sv.y;
        } else {
            const float4 sv = *reinterpret_cast<const float4 *>(ps);
            op.s[t][0] = sv.x;
            op.s[t][1] = sv.y;
            op.s[t][2] = sv.z;
            op.s[t][3] = sv.w;
        }
    }
#pragma unroll
    for (int rt = 0; rt < L::kRTW; ++rt) {
        const uint32_t *pw = reinterpret_cast<const uint32_t *>(slot + o.b + rt * 16 * kRowChunk);
        op.w[rt][0] = pw[0];
        op.w[rt][1] = pw[1];
        op.w[rt][2] = pw[2];
        op.d[rt] = *reinterpret_cast<const uint16_t *>(slot + o.d + rt * 16 * kRowChunk);
    }
}

// Where a lane's MFMA results belong, for the block-sum export: its weight row
// in the workgroup's range (first row tile of the wave; tile rt adds 16 rt) and
// its first activation row (first tile of the wave; tile t adds 16 t / WORDS).
struct SumsLane {
    int row;
    int rcount;
    uint32_t r0;
    int ar;
};

// One MFMA result of block blk to the export.  Two-word tiles: the lane holds
// (S_hi, S_lo) of activation rows ar and ar + 1; one-word tiles: S_hi of rows
// ar .. ar + 3.  A one-word stack in the two-word layout exports S_hi only.
template <int WORDS>
__device__ __forceinline__ void export_sums(const MmaArgs &a, const v4i &sum, int row, const SumsLane &sl, int ar,
                                            int blk) {
    if (row >= sl.rcount) return;
    const int64_t n = static_cast<int64_t>(sl.r0) + row;
    if constexpr (WORDS == 2) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            if (ar + i >= a.rows) continue;
            int32_t *o = a.sums + ((static_cast<int64_t>(ar + i) * a.sums_ld + n) * a.nb + blk) * a.sums_words;
            o[0] = sum[2 * i];
            if (a.sums_words == 2) o[1] = sum[2 * i + 1];
        }
    } else {
#pragma unroll
        for (int v = 0; v < 4; ++v)
            if (ar + v < a.rows) a.sums[(static_cast<int64_t>(ar + v) * a.sums_ld + n) * a.nb + blk] = sum[v];
    }
}

// The math of one block for this wave: realign the weight windows, one MFMA
// per (row tile, activation tile), and each term (d * s) * T into f64.
// SUMS: also export every MFMA result (block blk).
template <int RT, int TT, int WORDS, int GR, int GA, int GB, bool SUMS>
__device__ __forceinline__ void math_block(const BlockOps<RT, TT, WORDS, GR, GA, GB> &op, uint32_t sel,
                                           double (&acc)[Layout<RT, TT, WORDS, GR, GA, GB>::kRTW][Layout<RT, TT, WORDS, GR, GA, GB>::kAT][Layout<RT, TT, WORDS, GR, GA, GB>::kVals],
                                           const MmaArgs &ma, const SumsLane &sl, int blk) {
    using L = Layout<RT, TT, WORDS, GR, GA, GB>;
    constexpr int AT = L::kAT;
    double s[AT][L::kVals];
#pragma unroll
    for (int t = 0; t < AT; ++t)
#pragma unroll
        for (int v = 0; v < L::kVals; ++v) s[t][v] = static_cast<double>(op.s[t][v]);
#pragma unroll
    for (int rt = 0; rt < L::kRTW; ++rt) {
        const uint32_t lo32 = __builtin_amdgcn_perm(op.w[rt][1], op.w[rt][0], sel);
        const uint32_t hi32 = __builtin_amdgcn_perm(op.w[rt][2], op.w[rt][1], sel);
        const long bop = static_cast<long>((static_cast<uint64_t>(hi32) << 32) | lo32);
        const double d = static_cast<double>(f16_bits_to_float(op.d[rt]));
#pragma unroll
        for (int t = 0; t < AT; ++t) {
            const v4i sum = __builtin_amdgcn_mfma_i32_16x16x32_i8(op.a[t], bop, v4i{0, 0, 0, 0}, 0, 0, 0);
            if constexpr (SUMS) export_sums<WORDS>(ma, sum, sl.row + 16 * rt, sl, sl.ar + t * (16 / WORDS), blk);
            if constexpr (WORDS == 2) {
                const int t0 = sum[0] * 128 + sum[1];
                const int t1 = sum[2] * 128 + sum[3];
                acc[rt][t][0] = __builtin_fma(d * s[t][0], static_cast<double>(t0), acc[rt][t][0]);
                acc[rt][t][1] = __builtin_fma(d * s[t][1], static_cast<double>(t1), acc[rt][t][1]);
            } else {
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    acc[rt][t][v] = __builtin_fma(d * s[t][v], static_cast<double>(sum[v]), acc[rt][t][v]);
            }
        }
    }
}

// Blocks offs[0..NB) of a slot (chunk blocks blk0 + offs[].j), in that order:
// every operand read first.
template <int RT, int TT, int WORDS, int GR, int GA, int GB, int NB, bool SUMS>
__device__ __forceinline__ void compute_blocks(const uint8_t *slot, const BlockOffsets (&offs)[NB],
                                               double (&acc)[Layout<RT, TT, WORDS, GR, GA, GB>::kRTW][Layout<RT, TT, WORDS, GR, GA, GB>::kAT][Layout<RT, TT, WORDS, GR, GA, GB>::kVals],
                                               const MmaArgs &ma, const SumsLane &sl, int blk0) {
    BlockOps<RT, TT, WORDS, GR, GA, GB> op[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) load_block<RT, TT, WORDS, GR, GA, GB>(slot, offs[j], op[j]);
    __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead of the math: the scheduler would sink them
#pragma unroll
    for (int j = 0; j < NB; ++j)
        math_block<RT, TT, WORDS, GR, GA, GB, SUMS>(op[j], offs[j].sel, acc, ma, sl, blk0 + offs[j].j);
}

// The last workgroup of a split range: total i = sum over parts s (in order) of
// parts[s * kTot + i], into red[i].  Thread t takes i = t, t + T, ...; it
// issues the agent-scope loads of a group of G of its totals (all KS parts of
// each, at most 16 loads) at once, so the combine costs one memory round trip
// per group instead of one per load.
template <int KS, int kTot, int T>
__device__ __forceinline__ void combine_parts(const double *parts, double *red) {
    constexpr int kPer = (kTot + T - 1) / T;
    constexpr int G = KS >= 16 ? 1 : 16 / KS;
    const int t = static_cast<int>(threadIdx.x);
#pragma unroll
    for (int j0 = 0; j0 < kPer; j0 += G) {
        double p[G][KS];
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const int i = t + (j0 + g) * T;
            if (j0 + g < kPer && i < kTot) {
#pragma unroll
                for (int s = 0; s < KS; ++s)
                    p[g][s] = __hip_atomic_load(parts + static_cast<size_t>(s) * kTot + i, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
            }
        }
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const int i = t + (j0 + g) * T;
            if (j0 + g < kPer && i < kTot) {
                double tot = p[g][0];
#pragma unroll
                for (int s = 1; s < KS; ++s) tot += p[g][s];
                red[i] = tot;
            }
        }
    }
}

// The shared-ring projection of one workgroup.  SPLIT: K split over a.ksplit
// workgroups per row range, partials combined in a.ks_part (launched as
// mma_split_kernel, so that mma_kernel carries none of it).
template <int RT, int TT, int WORDS, int GR, int GA, int GB, bool SUMS, bool SPLIT>
__device__ __forceinline__ void mma_body(const MmaArgs &a) {
    static_assert(!SPLIT || !SUMS, "the block-sum export runs unsplit");
    using L = Layout<RT, TT, WORDS, GR, GA, GB>;
    constexpr int W = L::W;
    constexpr int AT = L::kAT;
    extern __shared__ __align__(16) uint8_t smem[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    constexpr int RTW = L::kRTW;
    const int ga = wave % GA, gr = (wave / GA) % GR, gb = wave / (GA * GR);
    const int ksplit = SPLIT ? a.ksplit : 1;
    const uint32_t range = blockIdx.x / static_cast<uint32_t>(ksplit);
    const int split = static_cast<int>(blockIdx.x - range * static_cast<uint32_t>(ksplit));
    const int kc0 = split * a.nchunks;  // this workgroup's first chunk
    const uint32_t r0 = range * static_cast<uint32_t>(a.rows_per_wg);
    const int rcount = static_cast<int>(min(static_cast<uint32_t>(a.rows_per_wg), a.n - r0));

    Rsrcs rs;
    rs.w = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(a.w), 0, a.w_bytes, kBufferDword3);
    const uint32_t act_bytes = static_cast<uint32_t>(a.rows) * a.k;
    rs.hi = __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t *>(a.hi), 0, act_bytes, kBufferDword3);
    rs.lo = WORDS == 2 ? __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t *>(a.lo), 0, act_bytes, kBufferDword3)
                       : rs.hi;
    rs.lo_oob = a.lo_oob;
    // the export passes no scales: an empty range reads zeros and touches nothing
    rs.s = SUMS ? __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t *>(a.hi), 0, 0, kBufferDword3)
                : __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(a.scale), 0,
                                                    static_cast<uint32_t>(a.rows) * a.nb * 4, kBufferDword3);
    const uint32_t base = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>((uintptr_t)(lds_ptr_t)smem));
    SumsLane sl;
    sl.row = gr * RTW * 16 + (lane & 15);
    sl.rcount = rcount;
    sl.r0 = r0;
    sl.ar = WORDS == 2 ? ga * AT * 8 + 2 * (lane >> 4) : ga * AT * 16 + 4 * (lane >> 4);

    uint32_t plan[L::kPerWave];
#pragma unroll
    for (int u = 0; u < L::kPerWave; ++u)
        plan[u] = plan_copy<RT, TT, WORDS, GR, GA, GB>(a, wave + W * u, lane, r0, rcount);
    BlockOffsets offs[L::kBlocksPerWave];
#pragma unroll
    for (int jj = 0; jj < L::kBlocksPerWave; ++jj)
        offs[jj] = block_offsets<RT, TT, WORDS, GR, GA, GB>(gb + GB * jj, ga * AT, gr * RTW, lane);

    double acc[RTW][AT][L::kVals];
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
        for (int t = 0; t < AT; ++t)
#pragma unroll
            for (int v = 0; v < L::kVals; ++v) acc[rt][t][v] = 0.0;

    // Prologue: chunks 0 .. kDepth-2 in flight.  Chunk 0 goes out alone first,
    // about half a microsecond ahead of the rest, so that the chip's first burst
    // of requests serves every workgroup's first chunk before any second one
    // (measured: 8 rows on 14336x4096, 16.6 -> 15.7 us; shorter or longer gaps
    // gained less).
#pragma unroll
    for (int c = 0; c < L::kDepth - 1; ++c) {
        if (c == 1) __builtin_amdgcn_s_sleep(20);  // 20 x 64 clocks
        issue_chunk<RT, TT, WORDS, GR, GA, GB>(rs, plan, base + c * L::kSlotBytes, c, a.nchunks, wave, kc0);
    }

    const bool more = wave < L::kCopies % W;  // this wave issues kPerWave copies per chunk, else kPerWaveLow
    int cur = 0;                 // slot of chunk c
    int nxt = L::kDepth - 1;     // slot of chunk c + kDepth - 1
    for (int c = 0; c < a.nchunks; ++c) {
        // this wave's copies of chunk c have landed
        if (more)
            wait_copies<L::kPerWave * (L::kDepth - 2)>();
        else
            wait_copies<L::kPerWaveLow * (L::kDepth - 2)>();
        ring_barrier();  // everyone's have; slot nxt is free
        issue_chunk<RT, TT, WORDS, GR, GA, GB>(rs, plan, base + nxt * L::kSlotBytes, c + L::kDepth - 1, a.nchunks,
                                           wave, kc0);
        const uint8_t *slot = smem + cur * L::kSlotBytes;
        compute_blocks<RT, TT, WORDS, GR, GA, GB, L::kBlocksPerWave, SUMS>(slot, offs, acc, a, sl,
                                                                           (kc0 + c) * kChunkBlocks);
        // the export's stores have completed before later waits count copies
        if constexpr (SUMS) wait_copies<0>();
        cur = cur + 1 == L::kDepth ? 0 : cur + 1;
        nxt = nxt + 1 == L::kDepth ? 0 : nxt + 1;
    }
    wait_copies<0>();  // the trailing copies read nothing but may still write the ring
    if constexpr (SUMS) return;
    ring_barrier();

    // Pairwise tree over the block groups of each (weight, activation) group:
    // at each level the upper half parks its accumulators in LDS and the lower
    // half adds them (fixed order).
    double *red = reinterpret_cast<double *>(smem);
    constexpr int kAccVals = RTW * AT * L::kVals;
    const int grp = ga + GA * gr;
#pragma unroll
    for (int half = GB / 2; half >= 1; half >>= 1) {
        if (gb >= half && gb < 2 * half) {
            double *dst = red + (grp + GA * GR * (gb - half)) * kAccVals * 64;
#pragma unroll
            for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
                for (int t = 0; t < AT; ++t)
#pragma unroll
                    for (int v = 0; v < L::kVals; ++v) dst[((rt * AT + t) * L::kVals + v) * 64 + lane] = acc[rt][t][v];
        }
        ring_barrier();
        if (gb < half) {
            const double *src = red + (grp + GA * GR * gb) * kAccVals * 64;
#pragma unroll
            for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
                for (int t = 0; t < AT; ++t)
#pragma unroll
                    for (int v = 0; v < L::kVals; ++v) acc[rt][t][v] += src[((rt * AT + t) * L::kVals + v) * 64 + lane];
        }
        ring_barrier();
    }
    // K split: these totals are one of ksplit partials of the row range.  Each
    // goes to the workspace as agent-scope atomic stores (written through this
    // XCD's L2 to the device-coherent level; no L2-wide write-back), completed
    // before the workgroup counts itself in.  The workgroup that counts last
    // reads every partial back at agent scope, adds them in split order (the
    // same bits whichever workgroup is last), writes the outputs as the
    // unsplit kernel does, and returns the counter to zero.
    if (SPLIT) {
        __shared__ int ks_last;
        constexpr int kTot = RT * TT * L::kVals * 64;
        const size_t range_part = static_cast<size_t>(range) * ksplit * kTot;
        if (gb == 0) {
#pragma unroll
            for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
                for (int t = 0; t < AT; ++t)
#pragma unroll
                    for (int v = 0; v < L::kVals; ++v) {
                        const int idx = (((gr * RTW + rt) * TT + ga * AT + t) * L::kVals + v) * 64 + lane;
                        __hip_atomic_store(a.ks_part + range_part + static_cast<size_t>(split) * kTot + idx,
                                           acc[rt][t][v], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    }
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        }
        __syncthreads();  // every partial of this workgroup has completed
        if (threadIdx.x == 0) {
            const uint32_t done = __hip_atomic_fetch_add(a.ks_count + range, 1u, __ATOMIC_RELAXED,
                                                         __HIP_MEMORY_SCOPE_AGENT);
            ks_last = done == static_cast<uint32_t>(ksplit - 1);
        }
        __syncthreads();
        if (!ks_last) return;
        // Every part is in the workspace, this workgroup's own included: add
        // them in part order into LDS, where the unsplit kernel parks its totals.
        const double *parts = a.ks_part + range_part;
        if (ksplit == 2)
            combine_parts<2, kTot, 64 * W>(parts, red);
        else if (ksplit == 4)
            combine_parts<4, kTot, 64 * W>(parts, red);
        else
            combine_parts<8, kTot, 64 * W>(parts, red);
        if (threadIdx.x == 0)
            __hip_atomic_store(a.ks_count + range, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else if (gb == 0) {
        // The waves of block group 0 hold the totals of their tiles; park them
        // as [rt][tile][v][lane] and let every wave write a share of the outputs.
#pragma unroll
        for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
            for (int t = 0; t < AT; ++t)
#pragma unroll
                for (int v = 0; v < L::kVals; ++v)
                    red[(((gr * RTW + rt) * TT + ga * AT + t) * L::kVals + v) * 64 + lane] = acc[rt][t][v];
    }
    ring_barrier();

    const double post = WORDS == 2 ? 1.0 / 128.0 : 1.0;
    const int q = lane >> 4;
    const int c16 = lane & 15;
    for (int p = wave; p < RT * TT; p += W) {
        const int rt = p / TT, t = p - (p / TT) * TT;
        const int row = rt * 16 + c16;
        if (row >= rcount) continue;
        const uint32_t n = r0 + row;
#pragma unroll
        for (int v = 0; v < L::kVals; ++v) {
            const int ar = WORDS == 2 ? t * 8 + 2 * q + v : t * 16 + 4 * q + v;
            if (ar >= a.rows) continue;
            const double tot = red[(p * L::kVals + v) * 64 + lane];
            const int64_t o = static_cast<int64_t>(ar) * a.ldy + n;
            const double res = a.residual ? static_cast<double>(a.residual[o]) : 0.0;
            a.y[o] = static_cast<float>(tot * post + res);
        }
    }
}

template <int RT, int TT, int WORDS, int GR, int GA, int GB, bool SUMS>
__global__ __launch_bounds__(64 * GR * GA * GB, 1) void mma_kernel(MmaArgs a) {
    mma_body<RT, TT, WORDS, GR, GA, GB, SUMS, false>(a);
}

template <int RT, int TT, int WORDS, int GR, int GA, int GB>
__global__ __launch_bounds__(64 * GR * GA * GB, 1) void mma_split_kernel(MmaArgs a) {
    mma_body<RT, TT, WORDS, GR, GA, GB, false, true>(a);
}

// ------------------------------------------------ one tile, wave-private rings
//
// A stack of one activation tile (up to 8 two-word or 16 one-word rows) against
// a 16-row weight tile, for short matrices where a workgroup owns a single tile.
// The shared-ring kernel above hands every chunk to all its waves through a
// barrier; with one tile each wave then has a single block of math per chunk,
// and the chunk's copy issue, its barrier and that block run in series.  Here
// the W waves split the chunks instead (wave w takes chunks w, w + W, ...):
// each copies its own chunks (weights, activation tile and scales, laid out as
// the shared slot is) into a private ring of P slots, waits for them by count
// and computes all eight blocks, with no barrier until the end.  The waves'
// partial sums are then added in wave order and each output rounded once.
template <int WORDS, int W, int P>
struct WaveLayout {
    using L = Layout<1, 1, WORDS, 1, 1, 1>;  // one wave issuing every copy of a chunk
    static constexpr int kVals = L::kVals;
    static constexpr int kRing = P * L::kSlotBytes;  // one wave's ring
    static constexpr int kLdsBytes = std::max(W * kRing, W * kVals * 64 * 8);
    static_assert(P >= 2 && P * L::kCopies <= 63, "outstanding copies exceed the vmcnt range");
    static_assert(W >= 1 && W <= 16, "at most 1024 threads");
};

template <int WORDS, int W, int P, bool SUMS>
__global__ __launch_bounds__(64 * W, 1) void mma_wave_kernel(MmaArgs a) {
    using WL = WaveLayout<WORDS, W, P>;
    using L = typename WL::L;
    constexpr int V = WL::kVals;
    extern __shared__ __align__(16) uint8_t smem[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t r0 = blockIdx.x * 16u;
    const int rcount = static_cast<int>(min(16u, a.n - r0));

    Rsrcs rs;
    rs.w = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(a.w), 0, a.w_bytes, kBufferDword3);
    const uint32_t act_bytes = static_cast<uint32_t>(a.rows) * a.k;
    rs.hi = __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t *>(a.hi), 0, act_bytes, kBufferDword3);
    rs.lo = WORDS == 2 ? __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t *>(a.lo), 0, act_bytes, kBufferDword3)
                       : rs.hi;
    rs.lo_oob = a.lo_oob;
    rs.s = SUMS ? __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t *>(a.hi), 0, 0, kBufferDword3)
                : __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(a.scale), 0,
                                                    static_cast<uint32_t>(a.rows) * a.nb * 4, kBufferDword3);
    SumsLane sl;
    sl.row = lane & 15;
    sl.rcount = rcount;
    sl.r0 = r0;
    sl.ar = WORDS == 2 ? 2 * (lane >> 4) : 4 * (lane >> 4);
    const uint8_t *ring = smem + wave * WL::kRing;
    const uint32_t ring_lds =
        __builtin_amdgcn_readfirstlane(static_cast<uint32_t>((uintptr_t)(lds_ptr_t)smem)) + wave * WL::kRing;

    uint32_t plan[L::kPerWave];
#pragma unroll
    for (int u = 0; u < L::kPerWave; ++u) plan[u] = plan_copy<1, 1, WORDS, 1, 1, 1>(a, u, lane, r0, rcount);
    BlockOffsets offs[kChunkBlocks];
#pragma unroll
    for (int j = 0; j < kChunkBlocks; ++j) offs[j] = block_offsets<1, 1, WORDS, 1, 1, 1>(j, 0, 0, lane);

    double acc[1][1][V];
#pragma unroll
    for (int v = 0; v < V; ++v) acc[0][0][v] = 0.0;

    // this wave's chunks: wave, wave + W, ...; copies past the last chunk read
    // nothing, so every step issues the same number and the counts stay exact
    const int mine = wave < a.nchunks ? (a.nchunks - wave + W - 1) / W : 0;
#pragma unroll
    for (int p = 0; p < P; ++p)
        issue_chunk<1, 1, WORDS, 1, 1, 1>(rs, plan, ring_lds + p * L::kSlotBytes, wave + W * p, a.nchunks, 0, 0);
    int slot = 0;
    for (int i = 0; i < mine; ++i) {
        wait_copies<(P - 1) * L::kCopies>();  // chunk i's copies have landed
        const uint8_t *s = ring + slot * L::kSlotBytes;
        compute_blocks<1, 1, WORDS, 1, 1, 1, kChunkBlocks, SUMS>(s, offs, acc, a, sl, (wave + W * i) * kChunkBlocks);
        // the export's stores have completed before later waits count copies
        if constexpr (SUMS) wait_copies<0>();
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the slot is read before it is refilled
        issue_chunk<1, 1, WORDS, 1, 1, 1>(rs, plan, ring_lds + slot * L::kSlotBytes, wave + W * (i + P), a.nchunks,
                                          0, 0);
        slot = slot + 1 == P ? 0 : slot + 1;
    }
    wait_copies<0>();  // the trailing copies read nothing but still write the ring
    if constexpr (SUMS) return;
    ring_barrier();    // every wave is done with its ring

    double *red = reinterpret_cast<double *>(smem);
#pragma unroll
    for (int v = 0; v < V; ++v) red[(wave * V + v) * 64 + lane] = acc[0][0][v];
    ring_barrier();
    if (wave != 0) return;
    const double post = WORDS == 2 ? 1.0 / 128.0 : 1.0;
    const int q = lane >> 4, c16 = lane & 15;
    if (c16 >= rcount) return;
    const uint32_t n = r0 + c16;
#pragma unroll
    for (int v = 0; v < V; ++v) {
        const int ar = WORDS == 2 ? 2 * q + v : 4 * q + v;
        if (ar >= a.rows) continue;
        double tot = red[v * 64 + lane];
        for (int w = 1; w < W; ++w) tot += red[(w * V + v) * 64 + lane];
        const int64_t o = static_cast<int64_t>(ar) * a.ldy + n;
        const double res = a.residual ? static_cast<double>(a.residual[o]) : 0.0;
        a.y[o] = static_cast<float>(tot * post + res);
    }
}

template <int WORDS, int W, int P, bool SUMS>
hipError_t run_wave(MmaArgs a, hipStream_t stream) {
    using WL = WaveLayout<WORDS, W, P>;
    if (WL::kLdsBytes > device_info().lds_per_block) return hipErrorInvalidConfiguration;
    a.rows_per_wg = 16;
    const uint32_t grid = (a.n + 15) / 16;
    hipLaunchKernelGGL((mma_wave_kernel<WORDS, W, P, SUMS>), dim3(grid), dim3(64 * W), WL::kLdsBytes, stream, a);
    return hipGetLastError();
}

template <int RT, int TT, int WORDS, int GR, int GA, int GB, bool SUMS>
hipError_t run(const MmaArgs &a, hipStream_t stream) {
    using L = Layout<RT, TT, WORDS, GR, GA, GB>;
    if (L::kLdsBytes > device_info().lds_per_block) return hipErrorInvalidConfiguration;
    const uint32_t grid = (a.n + a.rows_per_wg - 1) / a.rows_per_wg;
    hipLaunchKernelGGL((mma_kernel<RT, TT, WORDS, GR, GA, GB, SUMS>), dim3(grid), dim3(64 * L::W), L::kLdsBytes,
                       stream, a);
    return hipGetLastError();
}

// grid: a.ksplit workgroups for each range of a.rows_per_wg rows
template <int RT, int TT, int WORDS, int GR, int GA, int GB>
hipError_t run_ksplit(const MmaArgs &a, hipStream_t stream) {
    using L = Layout<RT, TT, WORDS, GR, GA, GB>;
    if (L::kLdsBytes > device_info().lds_per_block) return hipErrorInvalidConfiguration;
    const uint32_t grid = (a.n + a.rows_per_wg - 1) / a.rows_per_wg * static_cast<uint32_t>(a.ksplit);
    hipLaunchKernelGGL((mma_split_kernel<RT, TT, WORDS, GR, GA, GB>), dim3(grid), dim3(64 * L::W), L::kLdsBytes,
                       stream, a);
    return hipGetLastError();
}

// Wave split per (weight tiles, activation tiles), measured.
//  - One or two activation tiles and four weight tiles: sixteen waves, one
//    weight tile each, four block groups (2-6% and 7-11% faster than the
//    earlier 2x1x4 and 1x2x4).
//  - Two activation tiles and two weight tiles: sixteen waves, one tile of
//    each, four block groups (5% faster than 1x2x4).
//  - Two activation tiles and one weight tile: sixteen waves, eight block
//    groups.
//  - Eight activation tiles: four tiles a wave, eight block groups (with one
//    or two weight tiles 5-7% faster than 1x4x4).
//  - Otherwise one weight group and, by activation tiles: one tile, eight
//    block groups; two, one tile a wave and four block groups; four, two tiles
//    a wave and eight block groups.
// Splitting the output tiles wider than this (fewer block groups, less operand
// reuse per wave) measured slower.
struct Split {
    int gr, ga, gb;
};
constexpr Split wave_split(int rt, int tt) {
    if (rt == 4 && (tt == 1 || tt == 2)) return Split{4, 1, 4};
    if (rt == 2 && tt == 2) return Split{2, 2, 4};
    if (tt == 8) return Split{1, 2, 8};
    if (rt == 1 && tt == 2) return Split{1, 2, 8};
    return Split{1, tt == 1 ? 1 : 2, tt == 2 ? 4 : 8};
}

template <int WORDS, int TT, int RT, bool SUMS>
hipError_t run_split(const MmaArgs &a, hipStream_t s) {
    constexpr Split sp = wave_split(RT, TT);
    return run<RT, TT, WORDS, sp.gr, sp.ga, sp.gb, SUMS>(a, s);
}

template <int WORDS, int TT, bool SUMS>
hipError_t by_rt(int rt, const MmaArgs &a, hipStream_t s) {
    if (rt == 1) return run_split<WORDS, TT, 1, SUMS>(a, s);
    if (rt == 2) return run_split<WORDS, TT, 2, SUMS>(a, s);
    return run_split<WORDS, TT, 4, SUMS>(a, s);
}

// Activation tiles a stack needs.
int act_tiles(int words, int rows) {
    const int per = 16 / words;
    const int t = (rows + per - 1) / per;
    return t <= 1 ? 1 : t <= 2 ? 2 : t <= 4 ? 4 : 8;
}

// The kernel and wave split for a call (shared by the projection and the
// block-sum export, so that the export runs the projection's kernel).
// One launch over n weight rows (under 1 GiB of weights).  sums: this launch's
// first row of the export, whose row stride is sums_ld.
template <bool SUMS>
hipError_t launch_mma_slice(int mode, const uint8_t *w, int64_t n, int64_t k, int rows, const int8_t *hi,
                            const int8_t *lo, const float *scale, const float *residual, float *y, int64_t ldy,
                            int32_t *sums, int64_t sums_ld, hipStream_t stream) {
    // One-word stacks of up to eight rows run in the two-word layout with their
    // lo words read as zeros: T = 128 S_hi is exact, the final 1/128 undoes the
    // factor (a power of two: the f64 sums carry the same bits scaled), and a
    // lane rescales two rows per product instead of four.
    const bool as_two_word = mode == 1 && rows <= 8;
    const int words = mode == 2 || as_two_word ? 2 : 1;
    const int64_t nb = k / kBlock;
    const int at = act_tiles(words, rows);
    const int cus = std::max(1, device_info().cus);
    int64_t per_wg = (n + cus - 1) / cus;
    per_wg = std::min<int64_t>(per_wg, 64);
    const int rt = per_wg <= 16 ? 1 : per_wg <= 32 ? 2 : 4;
    MmaArgs a;
    a.w = w;
    a.hi = hi;
    a.lo = as_two_word ? hi : lo;
    a.lo_oob = as_two_word ? kOob : 0u;
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
    a.sums = sums;
    a.sums_ld = sums_ld;
    a.sums_words = mode == 2 ? 2 : 1;
    a.ksplit = 1;
    a.ks_part = nullptr;
    a.ks_count = nullptr;
    if (at == 1 && rt <= kWaveMaxRt) {
        if (words == 2) return run_wave<2, kWaveWaves, kWaveDepth, SUMS>(a, stream);
        return run_wave<1, kWaveWaves, kWaveDepth, SUMS>(a, stream);
    }
    if (words == 2) {
        switch (at) {
            case 1: return by_rt<2, 1, SUMS>(rt, a, stream);
            case 2: return by_rt<2, 2, SUMS>(rt, a, stream);
            case 4: return by_rt<2, 4, SUMS>(rt, a, stream);
            default: return by_rt<2, 8, SUMS>(rt, a, stream);
        }
    }
    switch (at) {
        case 1: return by_rt<1, 1, SUMS>(rt, a, stream);
        case 2: return by_rt<1, 2, SUMS>(rt, a, stream);
        default: return by_rt<1, 4, SUMS>(rt, a, stream);
    }
}

// The projection (or its block-sum export) over all n weight rows: launches
// over row slices of under 1 GiB of weights each (buffer offsets stay below
// 2^31), each reading its rows once; y, residual and the export are addressed
// with the whole call's row strides.
template <bool SUMS>
hipError_t launch_mma_impl(int mode, const uint8_t *w, int64_t n, int64_t k, int rows, const int8_t *hi,
                           const int8_t *lo, const float *scale, const float *residual, float *y, int64_t ldy,
                           int32_t *sums, hipStream_t stream) {
    const int64_t nb = k / kBlock;
    const int64_t row_bytes = nb * kBlockBytes;
    const int64_t slice = std::max<int64_t>(16, (kMaxMmaWeightBytes / row_bytes) / 16 * 16);
    const int64_t words = mode == 2 ? 2 : 1;
    for (int64_t n0 = 0; n0 < n; n0 += slice) {
        const int64_t ns = std::min(slice, n - n0);
        const hipError_t e = launch_mma_slice<SUMS>(mode, w + n0 * row_bytes, ns, k, rows, hi, lo, scale,
                                                    residual ? residual + n0 : nullptr, y ? y + n0 : nullptr, ldy,
                                                    sums ? sums + n0 * nb * words : nullptr, n, stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// ------------------------------------------- K split over workgroups (workspace)
//
// On a matrix of at most 16 rows per CU the dispatch above gives each
// workgroup one 16-row tile, so every workgroup copies the whole stack: as many
// bytes as its weights at 8 two-word rows of a long K, and two to eight times
// that for taller stacks; and a matrix of fewer than 16 rows per CU leaves CUs
// idle.  With a caller workspace the same stack runs instead on the shared
// ring with 64-row ranges and K split over ksplit workgroups per range
// (ranges x ksplit at most the CU count): each workgroup copies 1/ksplit of the
// stack.  The last workgroup of a range to finish reads every partial back and
// adds them: its partial written through, the counter, then the loads of all
// partials, one memory round trip each (a few for the widest stacks).
//
// When it pays (graphs of 20 launches, unsplit against split, two-word unless
// noted):
//  - Not when each workgroup gets fewer than 7 chunks: 4096 x 4096 loses at
//    every height (8 rows 7.3 against 9.0 us, 64 rows 19.5 against 24.8), as
//    do 2048 x 4096 and 1024 x 4096 beyond 9-32 rows.
//  - Stacks of two or more activation tiles (9+ two-word, 17+ one-word rows),
//    where the unsplit kernel is the shared ring with 16-row workgroups: 4096 x
//    14336 16 rows 25.7 against 21.2 us, 32 rows 39.3 against 28.4, 64 rows
//    58.2 against 47.5; one-word 32 rows 29.8 against 24.7; 4096 x 8192 16
//    rows 15.6 against 14.5.
//  - Matrices of at most 8 rows per CU (half the CUs idle unsplit), at any
//    height, where the split spans at least half the CUs: 2048 x 14336 8 rows
//    13.9 against 11.3, 1024 x 14336 13.2 against 10.4; not 512 x 14336 (64
//    workgroups), 2-6 rows 9.2-9.4 against 9.6-9.7.
//  - One tile on a full chip only for a large stack: 4096 x 14336 8 rows
//    (224 KB) 16.1 both ways, 2-6 rows about 1 us slower split, one-word 9-12
//    rows 1 us slower; 4096 x 28672 8 rows (448 KB) 29.5 against 27.4.
// Inside these rules one case measured slower split: 4096 x 8192 at 48-64
// one-word rows (23.4-23.8 against 24.9-25.3 us).
//
// The ranges' partials meet in the workspace: the counters (split_count_bytes:
// one u32 per 16-row tile of the tallest matrix that splits, which covers the
// ranges of every split kernel), then f64 partials [ranges][ksplit][4 * TT *
// kVals * 64].  The counters sit where no call's partials go, so one workspace
// serves calls of any shape.

constexpr int kSplitMinChunks = 7;                    // chunks per workgroup of a split
constexpr int64_t kSplitMinStackBytes = 400 * 1024;  // rows x words x k of a one-tile stack on a full chip

struct KsPlan {
    int words = 0;           // words of the layout (one-word stacks of up to 8 rows run two-word)
    int tt = 0;              // activation tiles
    int ksplit = 1;          // 1: no split for this stack
    int64_t ranges = 0;
    int64_t count_bytes = 0;
    int64_t bytes = 0;
};

KsPlan ks_plan(int mode, int64_t n, int64_t k, int rows) {
    KsPlan p;
    if ((mode != 1 && mode != 2) || n < 1 || rows < 1 || rows > 64) return p;
    const bool as_two_word = mode == 1 && rows <= 8;
    const int words = mode == 2 || as_two_word ? 2 : 1;
    const int64_t nb = k / kBlock;
    const int64_t cus = std::max(1, device_info().cus);
    if (nb % kChunkBlocks != 0 || n * nb * kBlockBytes >= kMaxMmaWeightBytes) return p;
    if (n > 16 * cus) return p;
    const int64_t ranges = (n + 63) / 64;
    int split = 1;
    for (int c : {8, 4, 2})
        if (ranges * c <= cus && nb % (kChunkBlocks * c) == 0) {
            split = c;
            break;
        }
    if (split == 1 || nb / (kChunkBlocks * split) < kSplitMinChunks) return p;
    const int tt = act_tiles(words, rows);
    // at most 8 rows per CU, split over at least half the CUs
    const bool idle_cus = n <= 8 * cus && 2 * ranges * split >= cus;
    const bool big_stack = int64_t(rows) * (mode == 2 ? 2 : 1) * k >= kSplitMinStackBytes;
    if (tt == 1 && !idle_cus && !big_stack) return p;
    const int64_t tot = 4 * tt * (words == 2 ? 2 : 4) * 64;  // RT * TT * kVals * 64 with RT = 4
    p.words = words;
    p.tt = tt;
    p.ksplit = split;
    p.ranges = ranges;
    p.count_bytes = split_count_bytes(static_cast<int>(cus));
    p.bytes = p.count_bytes + ranges * split * tot * 8;
    return p;
}

template <int WORDS, int TT>
hipError_t run_ksplit_tt(const MmaArgs &a, hipStream_t stream) {
    constexpr Split sp = wave_split(4, TT);
    return run_ksplit<4, TT, WORDS, sp.gr, sp.ga, sp.gb>(a, stream);
}

hipError_t launch_mma_ksplit_impl(int mode, const uint8_t *w, int64_t n, int64_t k, int rows, const int8_t *hi,
                                  const int8_t *lo, const float *scale, const float *residual, float *y,
                                  int64_t ldy, void *workspace, hipStream_t stream) {
    const KsPlan p = ks_plan(mode, n, k, rows);
    if (p.ksplit <= 1 || !workspace) return hipErrorInvalidValue;
    const bool as_two_word = p.words == 2 && mode == 1;
    const int64_t nb = k / kBlock;
    MmaArgs a;
    a.w = w;
    a.hi = hi;
    a.lo = as_two_word ? hi : lo;
    a.lo_oob = as_two_word ? kOob : 0u;
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
    a.rows_per_wg = 64;
    a.nchunks = static_cast<int>(nb / kChunkBlocks / p.ksplit);
    a.sums = nullptr;
    a.sums_ld = n;
    a.sums_words = mode == 2 ? 2 : 1;
    a.ksplit = p.ksplit;
    a.ks_count = static_cast<uint32_t *>(workspace);
    a.ks_part = reinterpret_cast<double *>(static_cast<uint8_t *>(workspace) + p.count_bytes);
    if (p.words == 2) {
        switch (p.tt) {
            case 1: return run_ksplit_tt<2, 1>(a, stream);
            case 2: return run_ksplit_tt<2, 2>(a, stream);
            case 4: return run_ksplit_tt<2, 4>(a, stream);
            default: return run_ksplit_tt<2, 8>(a, stream);
        }
    }
    switch (p.tt) {
        case 1: return run_ksplit_tt<1, 1>(a, stream);
        case 2: return run_ksplit_tt<1, 2>(a, stream);
        default: return run_ksplit_tt<1, 4>(a, stream);
    }
}

}  // namespace
}  // namespace q8
