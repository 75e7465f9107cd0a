/*
 * Seeded synthetic-input generator.
 *
 * This file draws random numbers and packs them into the storage formats the
 * decode path consumes (u8 codes with bf16 group scale/bias, bf16 and fp32
 * tensors).  It holds none of the decode arithmetic: both the CPU oracle and
 * the GPU path receive the bytes it writes and nothing else from it.
 *
 * Randomness: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random
 * numbers: as easy as 1, 2, 3", SC'11), a counter-based generator, so element
 * i of a tensor depends only on (key, i) and every thread count gives the same
 * bytes.  Normals come from the Box-Muller transform in double precision.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#define PHILOX_M0 0xD2511F53u
#define PHILOX_M1 0xCD9E8D57u
#define PHILOX_W0 0x9E3779B9u
#define PHILOX_W1 0xBB67AE85u

typedef struct { uint32_t v[4]; } ctr4;

static inline void mulhilo(uint32_t a, uint32_t b, uint32_t* hi, uint32_t* lo) {
    uint64_t p = (uint64_t)a * (uint64_t)b;
    *hi = (uint32_t)(p >> 32);
    *lo = (uint32_t)p;
}

/* Philox4x32 with 10 rounds: counter (c0..c3), key (k0, k1). */
static inline ctr4 philox4x32_10(ctr4 c, uint32_t k0, uint32_t k1) {
    for (int r = 0; r < 10; ++r) {
        uint32_t hi0, lo0, hi1, lo1;
        mulhilo(PHILOX_M0, c.v[0], &hi0, &lo0);
        mulhilo(PHILOX_M1, c.v[2], &hi1, &lo1);
        ctr4 n;
        n.v[0] = hi1 ^ c.v[1] ^ k0;
        n.v[1] = lo1;
        n.v[2] = hi0 ^ c.v[3] ^ k1;
        n.v[3] = lo0;
        c = n;
        k0 += PHILOX_W0;
        k1 += PHILOX_W1;
    }
    return c;
}

static inline ctr4 block_at(uint64_t key, uint64_t blk) {
    ctr4 c;
    c.v[0] = (uint32_t)blk;
    c.v[1] = (uint32_t)(blk >> 32);
    c.v[2] = 0x51ED5EEDu;
    c.v[3] = 0;
    return philox4x32_10(c, (uint32_t)key, (uint32_t)(key >> 32));
}

/* open interval (0, 1) */
static inline double u01(uint32_t r) { return ((double)r + 0.5) * (1.0 / 4294967296.0); }

/* Four standard normals from one Philox block via two Box-Muller pairs. */
static inline void normals4(uint64_t key, uint64_t blk, double z[4]) {
    ctr4 r = block_at(key, blk);
    const double two_pi = 6.283185307179586476925286766559;
    for (int p = 0; p < 2; ++p) {
        double rad = sqrt(-2.0 * log(u01(r.v[2 * p])));
        double ang = two_pi * u01(r.v[2 * p + 1]);
        z[2 * p] = rad * cos(ang);
        z[2 * p + 1] = rad * sin(ang);
    }
}

/* Round-to-nearest-even fp32 -> bf16 bits; NaN -> canonical quiet NaN. */
static inline uint16_t bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return 0x7FC0;
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

static inline float bf16_val(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* 64-bit FNV-1a of a tensor name, folded with the run seed. */
uint64_t synth_key(const char* name, uint64_t seed) {
    uint64_t h = 0xCBF29CE484222325ull;
    for (const unsigned char* p = (const unsigned char*)name; *p; ++p) {
        h ^= *p;
        h *= 0x100000001B3ull;
    }
    h ^= seed * 0x9E3779B97F4A7C15ull;
    h ^= h >> 29;
    return h;
}

/* out[i] = mean + std * N(0,1)_i  (fp32) */
void synth_normal_f32(uint64_t key, uint64_t n, double mean, double std, float* out) {
    int64_t nblk = (int64_t)((n + 3) / 4);
#pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < nblk; ++b) {
        double z[4];
        normals4(key, (uint64_t)b, z);
        for (int j = 0; j < 4; ++j) {
            uint64_t i = (uint64_t)b * 4 + j;
            if (i < n) out[i] = (float)(mean + std * z[j]);
        }
    }
}

/* out[i] = bf16(mean + std * N(0,1)_i) */
void synth_normal_bf16(uint64_t key, uint64_t n, double mean, double std, uint16_t* out) {
    int64_t nblk = (int64_t)((n + 3) / 4);
#pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < nblk; ++b) {
        double z[4];
        normals4(key, (uint64_t)b, z);
        for (int j = 0; j < 4; ++j) {
            uint64_t i = (uint64_t)b * 4 + j;
            if (i < n) out[i] = bf16_rne((float)(mean + std * z[j]));
        }
    }
}

/* out[i] = lo + (hi - lo) * U(0,1)_i  (fp32) */
void synth_uniform_f32(uint64_t key, uint64_t n, double lo, double hi, float* out) {
    int64_t nblk = (int64_t)((n + 3) / 4);
#pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < nblk; ++b) {
        ctr4 r = block_at(key, (uint64_t)b);
        for (int j = 0; j < 4; ++j) {
            uint64_t i = (uint64_t)b * 4 + j;
            if (i < n) out[i] = (float)(lo + (hi - lo) * u01(r.v[j]));
        }
    }
}

/* out[i] = bf16(lo + (hi - lo) * U(0,1)_i) */
void synth_uniform_bf16(uint64_t key, uint64_t n, double lo, double hi, uint16_t* out) {
    int64_t nblk = (int64_t)((n + 3) / 4);
#pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < nblk; ++b) {
        ctr4 r = block_at(key, (uint64_t)b);
        for (int j = 0; j < 4; ++j) {
            uint64_t i = (uint64_t)b * 4 + j;
            if (i < n) out[i] = bf16_rne((float)(lo + (hi - lo) * u01(r.v[j])));
        }
    }
}

/* bf16 rounding of an existing fp32 buffer (for inputs stored as bf16). */
void synth_f32_to_bf16(const float* in, uint64_t n, uint16_t* out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < (int64_t)n; ++i) out[i] = bf16_rne(in[i]);
}

/*
 * Synthetic affine 8-bit weights, groups of 64 along a row:
 *   w ~ N(0, std) in fp32, per group s = bf16((max - min) / 255), b = bf16(min),
 *   q = clamp(rint((w - b) / s), 0, 255).
 * Only (q, s, b) are written; w is discarded.  rows x k, k a multiple of 64.
 */
void synth_quant_g64(uint64_t key, uint64_t rows, uint64_t k, double std,
                     uint8_t* codes, uint16_t* scales, uint16_t* biases) {
    const uint64_t groups = k / 64;
    const int64_t total_groups = (int64_t)(rows * groups);
#pragma omp parallel for schedule(static)
    for (int64_t gi = 0; gi < total_groups; ++gi) {
        uint64_t base = (uint64_t)gi * 64; /* row-major: group gi covers [base, base+64) */
        float w[64];
        for (int b = 0; b < 16; ++b) {
            double z[4];
            normals4(key, base / 4 + (uint64_t)b, z);
            for (int j = 0; j < 4; ++j) w[b * 4 + j] = (float)(std * z[j]);
        }
        float mn = w[0], mx = w[0];
        for (int j = 1; j < 64; ++j) {
            if (w[j] < mn) mn = w[j];
            if (w[j] > mx) mx = w[j];
        }
        uint16_t sb = bf16_rne((mx - mn) / 255.0f);
        uint16_t bb = bf16_rne(mn);
        float s = bf16_val(sb), bias = bf16_val(bb);
        for (int j = 0; j < 64; ++j) {
            float t = (s > 0.0f) ? rintf((w[j] - bias) / s) : 0.0f;
            if (t < 0.0f) t = 0.0f;
            if (t > 255.0f) t = 255.0f;
            codes[base + j] = (uint8_t)t;
        }
        scales[gi] = sb;
        biases[gi] = bb;
    }
}
