/*
 * q8ref.c -- the CPU oracle of the Q8_0 projection.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg load this library.  The GPU library neither links, includes
 * nor calls anything here, and nothing here comes from the GPU library: the two
 * share no source, header, table or helper.
 *
 * Plain, slow, obviously correct.  Scalar loops; the only parallelism is an
 * OpenMP loop over independent output rows, which changes no value.  Build with
 * gcc -O2 -ffp-contract=off (no fast-math): every float expression below rounds
 * exactly as written, in IEEE-754 single or double precision.
 *
 * What is computed (sources: the logicaffeine_compile rustdoc pages
 * "codegen_cuda::lane", "model::author" and "spatial::streamed"):
 *
 *  - Q8_0 weights.  A projection's weight is stored as int8 values in blocks
 *    with one scale per block (model::author page, description: the .q/.s
 *    files); the product consumes those bytes as stored (spatial::streamed page,
 *    description, the paragraph on a weight moving as it is stored; lane page,
 *    description: quantized projections consumed straight from the checkpoint).  A block is 32 consecutive
 *    values of one output row with one binary16 scale, laid out as 34 bytes:
 *    the scale (little-endian) then the 32 int8 values.
 *  - Activation numerics, the lane's `activations` knob (lane page,
 *    description): f32 activations with f64 sums; a one-word int8 block
 *    quantization (llama.cpp's form); the default two-word ~14-bit int8 form.
 *    Readings taken where the page gives no formula are listed at each function.
 *
 * Parity unpinned: none.  Every function below is pinned by tests against
 * hand-worked blocks, closed forms, invariants, brute force or a library routine.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define Q8_BLOCK 32
#define Q8_BLOCK_BYTES 34

/* ---------------------------------------------------------------- helpers */

/* Round half away from zero: C's round() (ISO C 7.12.9.6). */
static float rha(float v) { return roundf(v); }

static int clamp127(float v) {
    if (v > 127.0f) return 127;
    if (v < -127.0f) return -127;
    return (int)v;
}

/* f32 -> IEEE-754 binary16, round to nearest, ties to even, subnormals kept,
 * overflow to infinity.  Written from the format's definition: find the
 * quantum (ulp) of the binary16 binade holding |x| (the subnormal quantum 2^-24
 * below 2^-14), round |x|/quantum to an integer with ties-to-even (rint in the
 * default rounding mode; the division by a power of two is exact in double),
 * then encode exponent and fraction. */
uint16_t q8ref_f16_bits(float x) {
    uint32_t xb;
    memcpy(&xb, &x, 4);
    uint16_t sign = (uint16_t)((xb >> 16) & 0x8000u);
    double a = fabs((double)x);
    if (isnan(x)) return (uint16_t)(sign | 0x7e00u);
    if (a == 0.0) return sign;
    int e;                                  /* a = m * 2^e, m in [0.5, 1) */
    frexp(a, &e);
    int unbiased = e - 1;                   /* a in [2^unbiased, 2^(unbiased+1)) */
    if (unbiased < -14) unbiased = -14;     /* subnormal range shares the 2^-24 quantum */
    double quantum = ldexp(1.0, unbiased - 10);
    double m = rint(a / quantum);           /* integer multiple of the quantum */
    if (m >= 2048.0) {                      /* rounded up into the next binade */
        m /= 2.0;
        unbiased += 1;
    }
    if (unbiased > 15) return (uint16_t)(sign | 0x7c00u);  /* overflow: infinity */
    if (m < 1024.0)                         /* subnormal (only when unbiased == -14) */
        return (uint16_t)(sign | (uint16_t)m);
    return (uint16_t)(sign | (uint16_t)((unbiased + 15) << 10) | (uint16_t)(m - 1024.0));
}

/* binary16 -> value (exact in float). */
float q8ref_f16_value(uint16_t h) {
    int exp = (h >> 10) & 0x1f;
    int frac = h & 0x3ff;
    double v;
    if (exp == 0) v = ldexp((double)frac, -24);
    else if (exp == 31) v = frac ? NAN : INFINITY;
    else v = ldexp((double)(1024 + frac), exp - 25);
    return (float)((h & 0x8000u) ? -v : v);
}

/* ------------------------------------------------------ weight quantization */

/* Q8_0 quantization of an f32 weight matrix w [n][k] into [n][k/32] 34-byte
 * blocks (model::author page, description: Q8_0 quants and block scales).
 * Per block: a = max |w_j| (exact); the scale is binary16(a / 127) (f32
 * division, correctly rounded, then round-to-nearest-even to binary16); each
 * value is w_j divided by the stored scale's value (f32 division), rounded half
 * away from zero and clamped to [-127, 127]; a zero scale gives all-zero values.
 * Reading: the values are divided by the stored binary16 scale (not by the f32
 * quotient), which is what bounds |scale*q - w| by half a scale step.
 * Returns 0, or -1 if k is not a multiple of 32. */
int q8ref_quantize_weights(const float *w, int64_t n, int64_t k, uint8_t *blocks) {
    if (k % Q8_BLOCK != 0 || n < 0 || k < 0) return -1;
    const int64_t nb = k / Q8_BLOCK;
#pragma omp parallel for schedule(static)
    for (int64_t row = 0; row < n; ++row) {
        for (int64_t b = 0; b < nb; ++b) {
            const float *src = w + row * k + b * Q8_BLOCK;
            uint8_t *dst = blocks + (row * nb + b) * Q8_BLOCK_BYTES;
            float amax = 0.0f;
            for (int j = 0; j < Q8_BLOCK; ++j)
                if (fabsf(src[j]) > amax) amax = fabsf(src[j]);
            float d32 = amax / 127.0f;
            uint16_t h = q8ref_f16_bits(d32);
            float dq = q8ref_f16_value(h);
            dst[0] = (uint8_t)(h & 0xff);
            dst[1] = (uint8_t)(h >> 8);
            for (int j = 0; j < Q8_BLOCK; ++j) {
                int q = (dq == 0.0f) ? 0 : clamp127(rha(src[j] / dq));
                dst[2 + j] = (uint8_t)(int8_t)q;
            }
        }
    }
    return 0;
}

/* Dequantized weights as doubles, [n][k]: scale * q, exact. */
int q8ref_dequantize_weights(const uint8_t *blocks, int64_t n, int64_t k, double *wd) {
    if (k % Q8_BLOCK != 0) return -1;
    const int64_t nb = k / Q8_BLOCK;
    for (int64_t row = 0; row < n; ++row)
        for (int64_t b = 0; b < nb; ++b) {
            const uint8_t *blk = blocks + (row * nb + b) * Q8_BLOCK_BYTES;
            double d = (double)q8ref_f16_value((uint16_t)(blk[0] | (blk[1] << 8)));
            for (int j = 0; j < Q8_BLOCK; ++j)
                wd[row * k + b * Q8_BLOCK + j] = d * (double)(int8_t)blk[2 + j];
        }
    return 0;
}

/* --------------------------------------------------- activation quantization */

/* Modes of the lane's `activations` knob (lane page, description). */
enum { MODE_F32 = 0, MODE_I8 = 1, MODE_I8X2 = 2 };

/* Activation quantization of x [rows][k] per 32-column block (lane page,
 * description: the one-word and two-word int8 activations; lane page, Modules,
 * kernels: an activation quantized for its projection).
 *   s    = max_j |x_j| / 127, kept in f32 (correctly rounded division)
 *   hi_j = clamp(rha(x_j / s))                           (one-word and two-word)
 *   lo_j = clamp(rha((fma(-s, hi_j, x_j) * 128) / s))    (two-word only)
 * and all-zero quants when s == 0.  Readings: the one-word form is llama.cpp's
 * block layout (int8 values plus one scale per 32) computed with a true
 * division; the two-word form is a second int8 word carrying the rounding
 * residual of the first at 1/128 of its step, on the same block scale, so
 * s*(hi + lo/128) approximates x to about 14 bits; the residual x - s*hi is
 * formed with one rounding (fused multiply-add).  Outputs: hi, lo [rows][k],
 * scale [rows][k/32].  lo may be NULL in one-word mode.  Returns 0, or -1 for a
 * bad mode or k not a multiple of 32. */
int q8ref_quantize_act(int mode, const float *x, int64_t rows, int64_t k, int8_t *hi, int8_t *lo,
                       float *scale) {
    if ((mode != MODE_I8 && mode != MODE_I8X2) || k % Q8_BLOCK != 0 || rows < 0) return -1;
    if (mode == MODE_I8X2 && lo == NULL) return -1;
    const int64_t nb = k / Q8_BLOCK;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t b = 0; b < nb; ++b) {
            const float *src = x + r * k + b * Q8_BLOCK;
            float amax = 0.0f;
            for (int j = 0; j < Q8_BLOCK; ++j)
                if (fabsf(src[j]) > amax) amax = fabsf(src[j]);
            float s = amax / 127.0f;
            scale[r * nb + b] = s;
            for (int j = 0; j < Q8_BLOCK; ++j) {
                int64_t idx = r * k + b * Q8_BLOCK + j;
                int h = (s == 0.0f) ? 0 : clamp127(rha(src[j] / s));
                hi[idx] = (int8_t)h;
                if (mode == MODE_I8X2) {
                    int l = 0;
                    if (s != 0.0f) {
                        float resid = fmaf(-s, (float)h, src[j]);
                        l = clamp127(rha((resid * 128.0f) / s));
                    }
                    lo[idx] = (int8_t)l;
                }
            }
        }
    return 0;
}

/* ------------------------------------------------------------ block sums */

/* Exact int32 block dot products of the integer modes (lane page, description:
 * the int8 activations against Q8_0 weights):
 *   S_hi[r][n][b] = sum_j q[n][b][j] * hi[r][32b + j]
 *   S_lo[r][n][b] = sum_j q[n][b][j] * lo[r][32b + j]   (two-word only)
 * Layout of sums: [rows][n][k/32][words], words = 1 (one-word) or 2 (hi, lo). */
int q8ref_block_sums(int mode, const uint8_t *blocks, int64_t n, int64_t k, int64_t rows,
                     const int8_t *hi, const int8_t *lo, int32_t *sums) {
    if ((mode != MODE_I8 && mode != MODE_I8X2) || k % Q8_BLOCK != 0) return -1;
    const int64_t nb = k / Q8_BLOCK;
    const int words = (mode == MODE_I8X2) ? 2 : 1;
#pragma omp parallel for schedule(static)
    for (int64_t row = 0; row < n; ++row)
        for (int64_t r = 0; r < rows; ++r)
            for (int64_t b = 0; b < nb; ++b) {
                const int8_t *q = (const int8_t *)(blocks + (row * nb + b) * Q8_BLOCK_BYTES + 2);
                int32_t sh = 0, sl = 0;
                for (int j = 0; j < Q8_BLOCK; ++j) {
                    sh += (int32_t)q[j] * (int32_t)hi[r * k + b * Q8_BLOCK + j];
                    if (words == 2) sl += (int32_t)q[j] * (int32_t)lo[r * k + b * Q8_BLOCK + j];
                }
                int32_t *out = sums + ((r * n + row) * nb + b) * words;
                out[0] = sh;
                if (words == 2) out[1] = sl;
            }
    return 0;
}

/* ------------------------------------------------------------ projection */

/* One output y[r][row] in double, with A = sum over blocks of |block term| +
 * |residual| (the scale of the rounding error any summation order can make).
 *   one-word: y = sum_b d_b * s_b * S_hi_b
 *   two-word: y = sum_b d_b * s_b * (S_hi_b + S_lo_b / 128)
 *   f32:      y = sum_b d_b * sum_j q_j * x_j            (every step in f64)
 * then y += residual (in f64).  d_b is the block's binary16 scale. */
static void project_one(int mode, const uint8_t *blocks, int64_t k, int64_t row, int64_t r,
                        const int8_t *hi, const int8_t *lo, const float *scale, const float *x,
                        const float *residual, int64_t n, double *out_y, double *out_a) {
    const int64_t nb = k / Q8_BLOCK;
    double y = 0.0, a = 0.0;
    for (int64_t b = 0; b < nb; ++b) {
        const uint8_t *blk = blocks + (row * nb + b) * Q8_BLOCK_BYTES;
        const int8_t *q = (const int8_t *)(blk + 2);
        double d = (double)q8ref_f16_value((uint16_t)(blk[0] | (blk[1] << 8)));
        double term;
        if (mode == MODE_F32) {
            double p = 0.0;
            for (int j = 0; j < Q8_BLOCK; ++j)
                p += (double)q[j] * (double)x[r * k + b * Q8_BLOCK + j];
            term = d * p;
        } else {
            int64_t sh = 0, sl = 0;
            for (int j = 0; j < Q8_BLOCK; ++j) {
                sh += (int64_t)q[j] * (int64_t)hi[r * k + b * Q8_BLOCK + j];
                if (mode == MODE_I8X2) sl += (int64_t)q[j] * (int64_t)lo[r * k + b * Q8_BLOCK + j];
            }
            double s = (double)scale[r * nb + b];
            double t = (mode == MODE_I8X2) ? (double)sh + (double)sl / 128.0 : (double)sh;
            term = d * s * t;
        }
        y += term;
        a += fabs(term);
    }
    if (residual) {
        double res = (double)residual[r * n + row];
        y += res;
        a += fabs(res);
    }
    *out_y = y;
    *out_a = a;
}

/* All outputs y[r][row] (rows x n, double) and their error scales A.
 * Inputs by mode: f32 uses x [rows][k]; the integer modes use hi (and lo for
 * two-word) [rows][k] and scale [rows][k/32].  residual [rows][n] may be NULL. */
int q8ref_project(int mode, const uint8_t *blocks, int64_t n, int64_t k, int64_t rows,
                  const int8_t *hi, const int8_t *lo, const float *scale, const float *x,
                  const float *residual, double *y, double *a) {
    if (mode < MODE_F32 || mode > MODE_I8X2 || k % Q8_BLOCK != 0) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t row = 0; row < n; ++row)
        for (int64_t r = 0; r < rows; ++r)
            project_one(mode, blocks, k, row, r, hi, lo, scale, x, residual, n,
                        &y[r * n + row], &a[r * n + row]);
    return 0;
}

/* The same for a list of (r, row) pairs only: outputs y[i], a[i] for
 * (r_idx[i], n_idx[i]).  For spot checks of shapes too large to project whole. */
int q8ref_project_at(int mode, const uint8_t *blocks, int64_t n, int64_t k, int64_t rows,
                     const int8_t *hi, const int8_t *lo, const float *scale, const float *x,
                     const float *residual, int64_t count, const int64_t *r_idx,
                     const int64_t *n_idx, double *y, double *a) {
    if (mode < MODE_F32 || mode > MODE_I8X2 || k % Q8_BLOCK != 0) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i) {
        if (r_idx[i] < 0 || r_idx[i] >= rows || n_idx[i] < 0 || n_idx[i] >= n) {
            y[i] = NAN;
            a[i] = NAN;
            continue;
        }
        project_one(mode, blocks, k, n_idx[i], r_idx[i], hi, lo, scale, x, residual, n, &y[i],
                    &a[i]);
    }
    return 0;
}

/* Brute force on tiny shapes: y[r][row] = sum_c wd[row][c] * v[r][c] by a direct
 * loop over columns in double, with no blocks.  Used with wd = the dequantized
 * weights (or the unquantized ones) and v = x or the dequantized activation. */
void q8ref_dense_matvec(const double *wd, int64_t n, int64_t k, int64_t rows, const double *v,
                        double *y) {
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t row = 0; row < n; ++row) {
            double acc = 0.0;
            for (int64_t c = 0; c < k; ++c) acc += wd[row * k + c] * v[r * k + c];
            y[r * n + row] = acc;
        }
}

/* Array forms of the scalar helpers, for the tests that sweep many inputs. */
void q8ref_f16_bits_array(const float *x, int64_t count, uint16_t *out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i) out[i] = q8ref_f16_bits(x[i]);
}

void q8ref_rha_array(const float *x, int64_t count, float *out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i) out[i] = rha(x[i]);
}

/* Threads the OpenMP loops above use, and a way to change that (for timing the
 * oracle on one thread and on all). */
#ifdef _OPENMP
#include <omp.h>
int q8ref_threads(void) { return omp_get_max_threads(); }
void q8ref_set_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }
#else
int q8ref_threads(void) { return 1; }
void q8ref_set_threads(int n) { (void)n; }
#endif
