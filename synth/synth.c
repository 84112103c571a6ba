/*
 * Seeded synthetic inputs for the Q8_0 projection: weight matrices, activation
 * stacks and residuals, plus the seeded choice of outlier rows and channels.
 *
 * This module is shared by the CPU oracle's tests and by the GPU library's tests
 * and benchmark.  It holds none of the projection's arithmetic: it only draws
 * numbers.
 *
 * Generator (published definitions, written from them):
 *   - SplitMix64 (G. Steele, D. Lea, C. Flood, "Fast splittable pseudorandom
 *     number generators", OOPSLA 2014): state advances by the golden-ratio
 *     increment 0x9e3779b97f4a7c15 and each state is passed through the
 *     variant-13 finaliser (shifts 30/27/31).  Because the state after i steps is
 *     seed + i*gamma, output i is a pure function of (seed, i): any sub-range of a
 *     stream can be drawn on its own, in parallel, with identical values.
 *   - uniform u in (0, 1]: the top 53 bits of an output, plus one, times 2^-53.
 *   - Box-Muller (G. Box, M. Muller, 1958): outputs 2p and 2p+1 give u1, u2;
 *     element 2p of the normal stream is sqrt(-2 ln u1) cos(2 pi u2) and element
 *     2p+1 is sqrt(-2 ln u1) sin(2 pi u2), in double, then times sigma, then
 *     rounded to float (round to nearest even).
 *   - distinct picks: a partial Fisher-Yates shuffle of 0..n-1 drawing the
 *     j-th swap partner as j + floor(u * (n - j)) from the uniform stream.
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC (no fast-math: libm's log/cos/sin in
 * double are used as they are).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

#define SM64_GAMMA 0x9e3779b97f4a7c15ULL

static inline uint64_t sm64_mix(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ULL;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebULL;
    return z ^ (z >> 31);
}

/* Output i (0-based) of the SplitMix64 stream seeded with `seed`. */
uint64_t synth_splitmix64_at(uint64_t seed, uint64_t i) {
    return sm64_mix(seed + (i + 1) * SM64_GAMMA);
}

/* Uniform in (0, 1] from output i. */
static inline double uniform_at(uint64_t seed, uint64_t i) {
    return (double)((synth_splitmix64_at(seed, i) >> 11) + 1) * 0x1.0p-53;
}

/* Normal-stream elements [offset, offset+count) of `seed`, times sigma, as float. */
void synth_normal_f32(uint64_t seed, int64_t offset, int64_t count, double sigma, float *out) {
    const double two_pi = 6.283185307179586476925286766559;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < count; ++t) {
        uint64_t e = (uint64_t)(offset + t);
        uint64_t pair = e >> 1;
        double u1 = uniform_at(seed, 2 * pair);
        double u2 = uniform_at(seed, 2 * pair + 1);
        double r = sqrt(-2.0 * log(u1));
        double v = (e & 1) ? r * sin(two_pi * u2) : r * cos(two_pi * u2);
        out[t] = (float)(v * sigma);
    }
}

/* `count` distinct indices of 0..n-1 drawn with a partial Fisher-Yates shuffle
 * on the uniform stream of `seed`.  Returns 0, or -1 if count > n or n < 1. */
int synth_pick(uint64_t seed, int64_t n, int64_t count, int64_t *out) {
    if (n < 1 || count < 0 || count > n) return -1;
    int64_t *perm = (int64_t *)malloc(sizeof(int64_t) * (size_t)n);
    if (!perm) return -1;
    for (int64_t i = 0; i < n; ++i) perm[i] = i;
    for (int64_t j = 0; j < count; ++j) {
        double u = uniform_at(seed, (uint64_t)j);          /* (0, 1] */
        int64_t span = n - j;
        int64_t off = (int64_t)floor((1.0 - u) * (double)span); /* [0, span) */
        if (off >= span) off = span - 1;
        int64_t k = j + off;
        int64_t tmp = perm[j];
        perm[j] = perm[k];
        perm[k] = tmp;
        out[j] = perm[j];
    }
    free(perm);
    return 0;
}

/* Multiply whole rows of a row-major [rows][cols] float matrix by `factor`
 * (exact when factor is a power of two). */
void synth_scale_rows(float *m, int64_t cols, const int64_t *rows, int64_t count, float factor) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i) {
        float *p = m + rows[i] * cols;
        for (int64_t c = 0; c < cols; ++c) p[c] *= factor;
    }
}

/* Multiply whole columns (channels) of a row-major [rows][cols] float matrix. */
void synth_scale_cols(float *m, int64_t rows, int64_t cols, const int64_t *chans, int64_t count,
                      float factor) {
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t i = 0; i < count; ++i) m[r * cols + chans[i]] *= factor;
}
