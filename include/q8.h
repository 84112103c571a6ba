/*
 * q8.h -- C ABI of libq8proj.so, the MI355X (gfx950) Q8_0 projection library.
 *
 * The projection is the wide product that a compiled decode step, a batched
 * decode step and a prefill chunk spend their bytes on: a matrix of Q8_0
 * weights times a stack of activation rows, every weight read once for the
 * whole stack (logicaffeine_compile, codegen_cuda::lane page, description;
 * model::author page, Functions: prefill, decode_batch).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All pointers are caller-owned device memory (the weight array may also be
 *    host memory the device maps: a kernel reads it through the same pointer and
 *    the result does not change; codegen_cuda::lane page, Modules: residence).
 *    The library allocates, frees and synchronizes nothing, and never reads
 *    device memory on the host (codegen_cuda::lane page, Modules: arena), so
 *    every call may be captured into a HIP graph.
 *  - `stream` is a hipStream_t (NULL: the null stream).  Work is enqueued
 *    asynchronously; results are ready when the stream is.
 *  - Arguments are validated before anything is enqueued; a failed check
 *    returns its named status and enqueues nothing (errors by name, as the
 *    lane's LaneError reports why a step does not compile; codegen_cuda::lane
 *    page, Enums: LaneError).  An empty problem (n == 0 or rows == 0) returns
 *    Q8_OK and enqueues nothing.  A launch failure returns Q8_E_HIP.  Device
 *    faults surface at the caller's next synchronization.
 *  - Inputs must be finite; NaN or infinity gives unspecified outputs.
 *
 * Data layout
 * -----------
 *  - Q8_0 weights W (n x k, out x in) are stored as in a checkpoint, read in
 *    place (codegen_cuda::lane page, description; model::author page,
 *    description: Q8_0 quants and block scales; spatial::streamed page,
 *    description: a weight is consumed as it is stored).  Row-major
 *    [n][k/32] blocks of 34 bytes: the block's binary16 scale d (little-endian),
 *    then 32 int8 values q.  Row n starts at byte n * (k/32) * 34.  The weight
 *    value is d * q.
 *  - Activation stacks are row-major [rows][k].  Quantized activations are
 *    hi and (two-word only) lo int8 [rows][k] and f32 block scales
 *    scale [rows][k/32].  Outputs and residuals are row-major f32 [rows][n].
 *  - k must be a positive multiple of 64 (whole blocks, dword-aligned rows).
 *
 * Numerics (codegen_cuda::lane page, description: the `activations` knob)
 * ----------------------------------------------------------------------
 *  Q8_ACT_F32  : f32 activations x; every product and sum in f64, rounded once
 *                to f32:  y = sum_b d_b * sum_j q_j * x_j  (+ residual).
 *  Q8_ACT_I8   : one int8 word per value (llama.cpp's block form): per
 *                32-column block s = max|x|/127 (f32), hi = rha(x/s).
 *                y = sum_b d_b * s_b * S_hi_b, S_hi_b = sum_j q_j * hi_j (int32).
 *  Q8_ACT_I8X2 : two words, ~14 bits (the lane's default): as one-word plus
 *                lo = rha((fma(-s, hi, x) * 128) / s) on the same scale.
 *                y = sum_b d_b * s_b * (S_hi_b + S_lo_b / 128).
 *  rha is round-half-away-from-zero, divisions are correctly rounded f32, an
 *  all-zero block gives zero quants.  The integer block sums are exact; the
 *  block terms are accumulated in f64 and each output is rounded once to f32.
 */
#ifndef Q8PROJ_Q8_H
#define Q8PROJ_Q8_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Activation numerics (the lane's `activations` knob). */
typedef enum {
    Q8_ACT_F32 = 0,  /* f32 activations, f64 sums */
    Q8_ACT_I8 = 1,   /* one int8 word */
    Q8_ACT_I8X2 = 2  /* two int8 words, the default */
} q8_act_mode;

/* Named results. */
typedef enum {
    Q8_OK = 0,
    Q8_E_NULL = 1,   /* a required pointer is NULL */
    Q8_E_SHAPE = 2,  /* negative size, k not a positive multiple of 64, or a size too large */
    Q8_E_ALIGN = 3,  /* a pointer breaks the alignment its argument requires */
    Q8_E_MODE = 4,   /* unknown mode, or a mode this entry point does not take */
    Q8_E_ALIAS = 5,  /* an output overlaps an input (other than y == residual exactly) */
    Q8_E_HIP = 6     /* the HIP runtime refused a launch */
} q8_status;

/* Q8_0-quantize an f32 weight matrix (off the projection's path: a checkpoint
 * already stores Q8_0; model::author page, description).  Per 32-block:
 * d = binary16(max|w| / 127) (round to nearest even), q = clamp(rha(w / d),
 * -127, 127) dividing by the stored binary16 value, q = 0 when d == 0.
 *   w      : f32 [n][k], 4-byte aligned.
 *   blocks : out, n * (k/32) * 34 bytes, 4-byte aligned, must not overlap w.
 * Errors: Q8_E_NULL, Q8_E_SHAPE, Q8_E_ALIGN, Q8_E_ALIAS, Q8_E_HIP. */
q8_status q8_quantize_weights(const float *w, int64_t n, int64_t k, void *blocks, void *stream);

/* Quantize an activation stack for the integer modes (codegen_cuda::lane page,
 * description: the one-word and two-word activations; Modules, kernels: an
 * activation quantized for its projection).
 *   mode   : Q8_ACT_I8 or Q8_ACT_I8X2 (Q8_ACT_F32 needs no quantization:
 *            Q8_E_MODE).
 *   x      : f32 [rows][k], 16-byte aligned.
 *   hi, lo : out, int8 [rows][k], 16-byte aligned; lo is required for
 *            Q8_ACT_I8X2 and ignored (may be NULL) for Q8_ACT_I8.
 *   scale  : out, f32 [rows][k/32], 4-byte aligned.
 * Outputs must not overlap x or each other.
 * Errors: Q8_E_NULL, Q8_E_SHAPE, Q8_E_ALIGN, Q8_E_MODE, Q8_E_ALIAS, Q8_E_HIP. */
q8_status q8_quantize_act(int mode, const float *x, int64_t rows, int64_t k, int8_t *hi, int8_t *lo,
                          float *scale, void *stream);

/* y = W x (+ residual) for ONE activation row: the decode step's projection
 * (codegen_cuda::lane page, description: quantized projections consumed straight
 * from the checkpoint).
 *   mode        : q8_act_mode.
 *   w           : Q8_0 blocks of an n x k matrix, 4-byte aligned (device or
 *                 host-mapped memory).
 *   hi, lo, scale : the row quantized by q8_quantize_act (integer modes;
 *                 hi/lo 16-byte aligned, lo only for Q8_ACT_I8X2); NULL in
 *                 Q8_ACT_F32.
 *   x           : f32 [k], 16-byte aligned.  Required in Q8_ACT_F32.  In an
 *                 integer mode, passing x with hi, lo and scale all NULL
 *                 quantizes the row inside the projection (the activation
 *                 quantization fused into its consumer; codegen_cuda::lane
 *                 page, Modules, kernels: fused forms): the result is bit for
 *                 bit that of q8_quantize_act then this call, and the
 *                 quantized row is not written out.  Every workgroup quantizes
 *                 the whole row again, so this pays off for small k (an LM
 *                 head) and costs time for large k.  A partial set of hi, lo,
 *                 scale is Q8_E_NULL.
 *   residual    : f32 [n] added to the result, or NULL.  4-byte aligned.
 *   y           : out, f32 [n], 4-byte aligned.  May be exactly `residual`
 *                 (in-place add); must not otherwise overlap any input.
 * Errors: Q8_E_NULL, Q8_E_SHAPE, Q8_E_ALIGN, Q8_E_MODE, Q8_E_ALIAS, Q8_E_HIP. */
q8_status q8_matvec(int mode, const void *w, int64_t n, int64_t k, const int8_t *hi, const int8_t *lo,
                    const float *scale, const float *x, const float *residual, float *y, void *stream);

/* Y = X W^T (+ residual) for a stack of `rows` activation rows, every weight
 * block read once per stack of up to 64 rows: a batched decode step (one row a
 * sequence) or a prefill chunk (model::author page, Functions: decode_batch,
 * prefill; codegen_cuda::lane page, description: prefill chunks of power-of-two
 * row counts).
 * Arguments as q8_matvec with [rows][...] stacks: hi/lo/x [rows][k],
 * scale [rows][k/32], residual and y [rows][n].  rows >= 1; stacks wider than
 * 64 rows are run as consecutive 64-row slices.  Kernels: integer stacks of
 * 2..64 rows on int8 MFMA tiles (or the GEMV for short stacks), f32 stacks of
 * 5..64 rows on f64 MFMA tiles (sums still exact products added in f64), up to
 * 4 rows on the GEMV; each slice streams the weights once.  Two cases fall back
 * to the GEMV 8 rows at a time, reading the weights once per 8 rows: integer
 * stacks whose k is not a multiple of 256 or whose weights or stack are not
 * 16-byte aligned, and f32 stacks with k above 2^22.  An integer-mode
 * stack given as x (hi, lo, scale NULL) is quantized inside the projection as
 * in q8_matvec, for at most 8 rows (one GEMV pass); a taller one is
 * Q8_E_SHAPE: quantize it once with q8_quantize_act (the result serves every
 * projection of the same input) and pass hi, lo and scale.  On a matrix of at
 * most 16 rows per CU, q8_matmul_rows_ws (below) is faster for most stacks.
 * Errors: Q8_E_NULL, Q8_E_SHAPE, Q8_E_ALIGN, Q8_E_MODE, Q8_E_ALIAS, Q8_E_HIP. */
q8_status q8_matmul_rows(int mode, const void *w, int64_t n, int64_t k, int64_t rows, const int8_t *hi,
                         const int8_t *lo, const float *scale, const float *x, const float *residual,
                         float *y, void *stream);

/* q8_matmul_rows with a caller workspace that lets stacks split K across
 * workgroups on short matrices: the batched decode step's and the prefill's
 * projections (model::author page, Functions: decode_batch, prefill) on a
 * matrix of at most 16 rows per CU, such as a layer's down projection (4096 x
 * 14336).  There q8_matmul_rows gives every workgroup one 16-row tile and the
 * whole stack, so each workgroup copies the stack (as many bytes as its
 * weights at 8 two-word rows of 14336, up to eight times that at 64 rows), and
 * a matrix of fewer rows leaves CUs idle.  This call gives each row range's K
 * to 2, 4 or 8 workgroups, which copy 1/2 .. 1/8 of the stack each (integer
 * modes: 64-row ranges on int8 matrix cores; f32 mode, 5..64 rows: 32-row
 * ranges on f64 matrix cores).  Their f64 partial sums meet in the workspace
 * and the last workgroup of a range to finish (told by an atomic counter) adds
 * them in split order, so the result does not depend on the order of arrival;
 * its f64 sums are added in another order than q8_matmul_rows's, so the two
 * may differ in the last bits of an output.  The combine costs the last
 * workgroup of each range a few memory round trips, so a slice splits only
 * where that measured to pay.  Integer modes: each part at least 7 chunks of
 * 256 columns, and either a stack of two or more activation tiles (over 8
 * two-word or 16 one-word rows), a matrix of at most 8 rows per CU whose split
 * spans at least half the CUs, or a stack of at least 400 KB (rows x k bytes,
 * twice in Q8_ACT_I8X2).  f32 mode: each part at least 16 blocks, and 128 for
 * stacks of up to 16 rows on matrices of more than 8 rows per CU.  Measured on
 * 4096 x 14336 (unsplit against split, varying by about 1 us between runs):
 * two-word 16 rows 25 against 21 us, 32 rows 36-38 against 27-28, 64 rows
 * 54 against 44; f32 16 rows 55 against 47, 64 rows 139 against 126; on 2048 x
 * 14336, two-word 8 rows 14 against 11.5, f32 64 rows 138 against 69.  Stacks
 * of more than 64 rows run as 64-row slices, one after another, each split or
 * not on its own.
 * Arguments as q8_matmul_rows, plus:
 *   workspace       : device memory, 16-byte aligned, of at least
 *                     q8_matmul_rows_workspace_bytes(mode, n, k, rows) bytes,
 *                     zero-filled by the caller before its first use.  It
 *                     starts with 32-bit counters, one for each 16-row tile
 *                     the tallest matrix that splits can have on this device
 *                     (16 rows per CU), which every call leaves at zero again;
 *                     the rest is scratch.  So one workspace, as large as the
 *                     largest call's, serves call after call of any shape
 *                     without clearing, but two calls in flight at once must
 *                     not share it.
 *   workspace_bytes : its size in bytes.
 * Where q8_matmul_rows_workspace_bytes is 0 (one row, f32 stacks under 5
 * rows, more than 16 rows per CU, no 64-row slice that splits by the rules
 * above, integer k not a multiple of 256, weights of 1 GiB or more), for an
 * integer stack given as x, and for slices q8_matmul_rows would not run on its
 * matrix-core kernels (16-byte alignment), the call or slice is
 * q8_matmul_rows's and the workspace is not read or written (it may be NULL
 * where no slice splits).
 * Errors: as q8_matmul_rows; with a workspace needed: Q8_E_NULL (none given),
 * Q8_E_ALIGN, Q8_E_SHAPE (workspace_bytes too small), Q8_E_ALIAS (workspace
 * overlapping an input or y). */
q8_status q8_matmul_rows_ws(int mode, const void *w, int64_t n, int64_t k, int64_t rows, const int8_t *hi,
                            const int8_t *lo, const float *scale, const float *x, const float *residual,
                            float *y, void *workspace, int64_t workspace_bytes, void *stream);

/* Bytes of the q8_matmul_rows_ws workspace for this call on the current device,
 * 0 where the call does not split K (or the arguments are out of range). */
int64_t q8_matmul_rows_workspace_bytes(int mode, int64_t n, int64_t k, int64_t rows);

/* y = W x (+ residual) for one activation row, and idx = argmax_i y[i] (the
 * lowest i among equal maxima) from the same launch: the LM head closing a
 * decode step (model::author page, Functions: the head reads the last row
 * only).  Arguments as q8_matvec (including x alone in an integer mode), plus:
 *   idx       : out, int32 (device), 4-byte aligned.
 *   workspace : device memory of q8_argmax_workspace_bytes(n) bytes, 16-byte
 *               aligned, zero-filled by the caller before its first use.  Its
 *               first 16 bytes hold a counter that every call leaves at zero
 *               again; the rest is scratch.  So one workspace serves call
 *               after call without clearing, but two calls in flight at once
 *               must not share it.
 * The arg-max is over the stored f32 y.  Every workgroup reduces its rows to a
 * partial in the workspace; the last one to finish, told by an atomic counter,
 * reduces the partials.  The order of arrival does not change the result.
 * Limits (else Q8_E_SHAPE): 1 <= n <= 2^31 - 1, weights at most 1 GiB, and the
 * row's staged activations within 64 KiB (k up to 30784 two-word, 58240
 * one-word, 16384 in f32 mode).  idx and the workspace must not overlap any other
 * argument (Q8_E_ALIAS).
 * Errors: Q8_E_NULL, Q8_E_SHAPE, Q8_E_ALIGN, Q8_E_MODE, Q8_E_ALIAS, Q8_E_HIP. */
q8_status q8_matvec_argmax(int mode, const void *w, int64_t n, int64_t k, const int8_t *hi, const int8_t *lo,
                           const float *scale, const float *x, const float *residual, float *y, int32_t *idx,
                           void *workspace, void *stream);

/* Bytes of the q8_matvec_argmax workspace for n weight rows on the current
 * device (0 if n is out of range). */
int64_t q8_argmax_workspace_bytes(int64_t n);

/* q8_matvec_argmax for callers that cannot allocate: code under HIP graph
 * capture, serving loops that may not call hipMalloc, harnesses that forbid
 * it.  Arguments, results and limits as q8_matvec_argmax, without the
 * workspace: the library uses a fixed 64 KiB device array of its own instead
 * (one per GPU, held until the process ends; its address is looked up once per
 * device, on the first call there).  Each call clears the array's counter with
 * a one-workgroup kernel on `stream`, then launches the projection; nothing is
 * allocated, freed or set with a memset, so the pair can be captured into a
 * graph.  Every call on one GPU shares that GPU's array: calls that overlap on
 * one GPU (other streams, other threads) race, and the caller must serialize
 * them.  Limit: q8_argmax_workspace_bytes(n) <= 65536 (n up to about 4.19
 * million rows on a 256-CU device), else Q8_E_SHAPE.
 * Errors: as q8_matvec_argmax; Q8_E_HIP also if the array's address cannot be
 * found. */
q8_status q8_matvec_argmax_noalloc(int mode, const void *w, int64_t n, int64_t k, const int8_t *hi,
                                   const int8_t *lo, const float *scale, const float *x, const float *residual,
                                   float *y, int32_t *idx, void *stream);

/* The exact int32 block dot products of the integer modes, for checking:
 *   sums[r][n][b][0] = sum_j q[n][b][j] * hi[r][32b+j]
 *   sums[r][n][b][1] = sum_j q[n][b][j] * lo[r][32b+j]   (Q8_ACT_I8X2 only)
 * computed by the kernel that q8_matmul_rows runs for the same stack (the
 * same 64-row slices and 8-row GEMV chunks, the GEMV or MFMA kernel and its
 * wave split, with the scales counted as 16-byte aligned), with that kernel's
 * block-sum export on: it writes each block's int32 sums where the projection
 * scales and accumulates them.  sums: out, int32 [rows][n][k/32][words],
 * 4-byte aligned.  Errors as q8_matmul_rows (Q8_ACT_F32: Q8_E_MODE). */
q8_status q8_block_sums(int mode, const void *w, int64_t n, int64_t k, int64_t rows, const int8_t *hi,
                        const int8_t *lo, int32_t *sums, void *stream);

/* Name of a status ("Q8_OK", "Q8_E_SHAPE", ...); "Q8_E_UNKNOWN" otherwise. */
const char *q8_status_name(int status);

/* Library version, major * 10000 + minor * 100 + patch. */
int q8_version(void);

#ifdef __cplusplus
}
#endif

#endif /* Q8PROJ_Q8_H */
