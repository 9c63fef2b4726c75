/*
 * Seeded synthetic inputs for the decode-step tests and benchmark.
 *
 * This file generates INPUTS only (weights, norm gains, prompt token ids and
 * optional synthetic KV-cache contents). It contains none of the decode-step
 * arithmetic: both the CPU oracle and the GPU library receive the arrays it
 * writes, byte for byte.
 *
 * Random numbers come from the counter-based generator Philox4x32-10
 * (J. Salmon, M. Moraes, R. Dror, D. Shaw, "Parallel random numbers: as easy
 * as 1, 2, 3", SC'11), keyed by (seed) with the counter (element block,
 * stream id).  Normal variates use the Box-Muller transform
 * (G. Box, M. Muller, Ann. Math. Statist. 29(2), 1958).  Because the value of
 * element i depends only on (seed, stream, i), any slice of any tensor can be
 * regenerated independently and in parallel.
 *
 * Storage: float32, or bfloat16 bits obtained by round-to-nearest-even of the
 * float64 draw (the upper 16 bits of an IEEE binary32 with RNE on the lower
 * 16; NaN is never produced here).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define PHILOX_M0 0xD2511F53u
#define PHILOX_M1 0xCD9E8D57u
#define PHILOX_W0 0x9E3779B9u
#define PHILOX_W1 0xBB67AE85u

static inline void philox4x32_10(uint32_t ctr[4], uint32_t k0, uint32_t k1) {
    for (int r = 0; r < 10; ++r) {
        uint64_t p0 = (uint64_t)PHILOX_M0 * ctr[0];
        uint64_t p1 = (uint64_t)PHILOX_M1 * ctr[2];
        uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        uint32_t n0 = hi1 ^ ctr[1] ^ k0;
        uint32_t n2 = hi0 ^ ctr[3] ^ k1;
        ctr[0] = n0; ctr[1] = lo1; ctr[2] = n2; ctr[3] = lo0;
        k0 += PHILOX_W0; k1 += PHILOX_W1;
    }
}

/* Exposed for the known-answer test of the generator itself. */
void synth_philox4x32_10(const uint32_t in_ctr[4], const uint32_t key[2], uint32_t out[4]) {
    uint32_t c[4] = {in_ctr[0], in_ctr[1], in_ctr[2], in_ctr[3]};
    philox4x32_10(c, key[0], key[1]);
    memcpy(out, c, sizeof c);
}

/* Four u32 words for block b of stream `stream` under `seed`. */
static inline void block_words(uint64_t seed, uint32_t stream, uint64_t b, uint32_t out[4]) {
    out[0] = (uint32_t)b; out[1] = (uint32_t)(b >> 32); out[2] = stream; out[3] = 0x6d6b7379u;
    philox4x32_10(out, (uint32_t)seed, (uint32_t)(seed >> 32));
}

/* u32 -> uniform double in the open interval (0, 1). */
static inline double u01(uint32_t x) { return ((double)x + 0.5) * (1.0 / 4294967296.0); }

/* The four standard-normal variates of block b (two Box-Muller pairs). */
static inline void block_normals(uint64_t seed, uint32_t stream, uint64_t b, double z[4]) {
    uint32_t w[4];
    block_words(seed, stream, b, w);
    const double two_pi = 6.283185307179586476925286766559;
    for (int p = 0; p < 2; ++p) {
        double r = sqrt(-2.0 * log(u01(w[2 * p])));
        double t = two_pi * u01(w[2 * p + 1]);
        z[2 * p] = r * cos(t);
        z[2 * p + 1] = r * sin(t);
    }
}

static inline uint16_t f64_to_bf16_rne(double v) {
    float f = (float)v; /* IEEE default rounding: to nearest even */
    uint32_t u;
    memcpy(&u, &f, 4);
    /* The float rounding may have landed exactly on a bf16 midpoint that the
       float64 value is not on; step one float ulp back toward v so the tie
       rule below only fires on true ties. */
    if ((u & 0xFFFFu) == 0x8000u && (double)f != v) u += (fabs(v) > fabs((double)f)) ? 1u : (uint32_t)-1;
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7FFFu + lsb;
    return (uint16_t)(u >> 16);
}

/*
 * Fill out[0..n) with mean + std * N(0,1) for elements [offset, offset+n) of
 * stream `stream`.  dtype 0 = float32, 1 = bfloat16 bits (uint16), 2 = int8
 * codes (the draw rounded to the nearest integer and clamped to [-127, 127]:
 * the code distribution of a weight-only INT8 matrix).
 */
void synth_normal(uint64_t seed, uint32_t stream, uint64_t offset, uint64_t n,
                  double mean, double std, int dtype, void *out) {
    if (n == 0) return;
    uint64_t b0 = offset >> 2, b1 = (offset + n - 1) >> 2;
    int64_t nb = (int64_t)(b1 - b0 + 1);
#pragma omp parallel for schedule(static)
    for (int64_t bi = 0; bi < nb; ++bi) {
        uint64_t b = b0 + (uint64_t)bi;
        double z[4];
        block_normals(seed, stream, b, z);
        for (int k = 0; k < 4; ++k) {
            uint64_t e = b * 4 + (uint64_t)k;
            if (e < offset || e >= offset + n) continue;
            double v = mean + std * z[k];
            uint64_t i = e - offset;
            if (dtype == 0) {
                ((float *)out)[i] = (float)v;
            } else if (dtype == 1) {
                ((uint16_t *)out)[i] = f64_to_bf16_rne(v);
            } else {
                double r = nearbyint(v);
                ((int8_t *)out)[i] = (int8_t)(r > 127.0 ? 127 : r < -127.0 ? -127 : (int)r);
            }
        }
    }
}

/* Uniform integers in [0, hi) for elements [offset, offset+n) of a stream. */
void synth_uniform_int(uint64_t seed, uint32_t stream, uint64_t offset, uint64_t n,
                       uint32_t hi, int32_t *out) {
    for (uint64_t i = 0; i < n; ++i) {
        uint64_t e = offset + i;
        uint32_t w[4];
        block_words(seed, stream, e >> 2, w);
        out[i] = (int32_t)(((uint64_t)w[e & 3] * (uint64_t)hi) >> 32);
    }
}

/* Uniform float32 values in [lo, hi) for elements [offset, offset+n) of a
   stream (per-row scales of the INT8 matrices). */
void synth_uniform_f32(uint64_t seed, uint32_t stream, uint64_t offset, uint64_t n, double lo, double hi,
                       float *out) {
    for (uint64_t i = 0; i < n; ++i) {
        uint64_t e = offset + i;
        uint32_t w[4];
        block_words(seed, stream, e >> 2, w);
        out[i] = (float)(lo + (hi - lo) * ((double)w[e & 3] * (1.0 / 4294967296.0)));
    }
}
