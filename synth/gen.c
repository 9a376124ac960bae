/*
 * Seeded synthetic input generator (inputs only: holds none of the MoE
 * method's arithmetic).  Every value is a pure function of
 * (seed, tag, element index), so any slice of any tensor -- one expert of
 * one layer, say -- can be produced on its own, in parallel, and both the
 * fp64 oracle and the GPU library receive byte-identical inputs.
 *
 * Stream definition
 *   key          = mix64(mix64(seed) + tag)                 (tag: 64-bit hash of a name)
 *   word(n)      = mix64(key + (n + 1) * 0x9E3779B97F4A7C15) (n-th SplitMix64 output)
 *   mix64        = the SplitMix64 finaliser (Steele, Lea & Flood, OOPSLA 2014;
 *                  constants as published by Vigna for splitmix64.c)
 * Normal pairs (Box-Muller, 1958): element 2n and 2n+1 use word(n):
 *   u1 = (hi32 + 0.5) / 2^32, u2 = (lo32 + 0.5) / 2^32
 *   z0 = sqrt(-2 ln u1) cos(2 pi u2), z1 = sqrt(-2 ln u1) sin(2 pi u2)
 * Outputs
 *   bf16: sigma*z in fp64, rounded once to bf16 (round to nearest, ties to even)
 *   f32 : sigma*z in fp64, rounded once to fp32 (C cast, round to nearest even)
 *   u8  : byte (i mod 8) of word(i / 8), little-endian byte order
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GOLDEN 0x9E3779B97F4A7C15ull

static inline uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

static inline uint64_t stream_key(uint64_t seed, uint64_t tag) {
    return mix64(mix64(seed) + tag);
}

static inline uint64_t word_at(uint64_t key, uint64_t n) {
    return mix64(key + (n + 1) * GOLDEN);
}

static inline void normal_pair(uint64_t w, double *z0, double *z1) {
    const double two32 = 4294967296.0;
    double u1 = ((double)(w >> 32) + 0.5) / two32;
    double u2 = ((double)(w & 0xFFFFFFFFull) + 0.5) / two32;
    double rad = sqrt(-2.0 * log(u1));
    double ang = 6.283185307179586476925286766559 * u2;
    *z0 = rad * cos(ang);
    *z1 = rad * sin(ang);
}

/* Round a double to the nearest bf16 (ties to even) and return its bits.
 * Values below the bf16 normal range are rounded on the subnormal grid. */
static inline uint16_t double_to_bf16_rne(double x) {
    if (x == 0.0) return signbit(x) ? 0x8000 : 0x0000;
    int e = ilogb(x);                 /* 2^e <= |x| < 2^(e+1) */
    if (e < -126) e = -126;           /* subnormal grid of bf16 */
    double m = nearbyint(ldexp(x, 7 - e));   /* default mode: nearest-even */
    double r = ldexp(m, e - 7);       /* exactly representable in bf16 (and fp32) */
    float f = (float)r;
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

void synth_normal_bf16(uint64_t seed, uint64_t tag, int64_t n, double sigma, uint16_t *out) {
    uint64_t key = stream_key(seed, tag);
    int64_t npairs = (n + 1) / 2;
#pragma omp parallel for schedule(static)
    for (int64_t p = 0; p < npairs; ++p) {
        double z0, z1;
        normal_pair(word_at(key, (uint64_t)p), &z0, &z1);
        out[2 * p] = double_to_bf16_rne(sigma * z0);
        if (2 * p + 1 < n) out[2 * p + 1] = double_to_bf16_rne(sigma * z1);
    }
}

void synth_normal_f32(uint64_t seed, uint64_t tag, int64_t n, double sigma, float *out) {
    uint64_t key = stream_key(seed, tag);
    int64_t npairs = (n + 1) / 2;
#pragma omp parallel for schedule(static)
    for (int64_t p = 0; p < npairs; ++p) {
        double z0, z1;
        normal_pair(word_at(key, (uint64_t)p), &z0, &z1);
        out[2 * p] = (float)(sigma * z0);
        if (2 * p + 1 < n) out[2 * p + 1] = (float)(sigma * z1);
    }
}

void synth_uniform_u8(uint64_t seed, uint64_t tag, int64_t n, uint8_t *out) {
    uint64_t key = stream_key(seed, tag);
    int64_t nwords = (n + 7) / 8;
#pragma omp parallel for schedule(static)
    for (int64_t w = 0; w < nwords; ++w) {
        uint64_t v = word_at(key, (uint64_t)w);
        for (int b = 0; b < 8 && 8 * w + b < n; ++b) out[8 * w + b] = (uint8_t)(v >> (8 * b));
    }
}

/* Raw 64-bit words, for integer draws made by the harness (e.g. picking experts). */
void synth_words(uint64_t seed, uint64_t tag, int64_t n, uint64_t *out) {
    uint64_t key = stream_key(seed, tag);
    for (int64_t i = 0; i < n; ++i) out[i] = word_at(key, (uint64_t)i);
}
