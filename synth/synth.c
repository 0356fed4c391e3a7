/*
 * Seeded synthetic inputs shared by the oracle and the GPU path.
 *
 * This file holds no arithmetic of the decode step itself: it only turns
 * (seed, stream, index) into pseudo-random numbers. Both sides of every
 * parity test read the same generated bits; neither side runs this code
 * as part of its computation.
 *
 * Generator: counter based, so the output does not depend on the thread
 * count or on chunking.
 *   key      = splitmix64(seed * 0x100000001B3 ^ splitmix64(stream))
 *   word(i)  = splitmix64(key + i)
 * splitmix64 is Steele, Lea and Flood's SplitMix64 finaliser ("Fast
 * splittable pseudorandom number generators", OOPSLA 2014).
 * Normals come in pairs from the Box-Muller transform (Box and Muller,
 * 1958) on two uniforms in (0, 1]: pair p uses word(2p) and word(2p+1).
 * Values are formed in double, rounded to float, then (for bf16) rounded
 * to nearest-even on the upper 16 bits.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

static inline uint64_t splitmix64(uint64_t z) {
    z += 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

static inline uint64_t stream_key(uint64_t seed, uint64_t stream) {
    return splitmix64(seed * 0x100000001B3ull ^ splitmix64(stream));
}

/* uniform in (0, 1] with 53 random bits */
static inline double u01(uint64_t w) { return ((double)(w >> 11) + 1.0) * (1.0 / 9007199254740992.0); }

static inline uint16_t f32_to_bf16_rne(float f) {
    uint32_t b;
    memcpy(&b, &f, 4);
    if ((b & 0x7F800000u) == 0x7F800000u && (b & 0x007FFFFFu)) return (uint16_t)((b >> 16) | 0x40u);
    b += 0x7FFFu + ((b >> 16) & 1u);
    return (uint16_t)(b >> 16);
}

static inline void normal_pair(uint64_t key, int64_t p, double* z0, double* z1) {
    double u1 = u01(splitmix64(key + (uint64_t)(2 * p)));
    double u2 = u01(splitmix64(key + (uint64_t)(2 * p + 1)));
    double r = sqrt(-2.0 * log(u1));
    double t = 6.283185307179586476925286766559 * u2;
    *z0 = r * cos(t);
    *z1 = r * sin(t);
}

#define CHUNK 65536

void synth_normal_f32(uint64_t seed, uint64_t stream, double mean, double std, int64_t n, float* out) {
    const uint64_t key = stream_key(seed, stream);
    const int64_t npairs = (n + 1) / 2;
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < npairs; c += CHUNK) {
        int64_t e = c + CHUNK < npairs ? c + CHUNK : npairs;
        for (int64_t p = c; p < e; ++p) {
            double z0, z1;
            normal_pair(key, p, &z0, &z1);
            out[2 * p] = (float)(mean + std * z0);
            if (2 * p + 1 < n) out[2 * p + 1] = (float)(mean + std * z1);
        }
    }
}

void synth_normal_bf16(uint64_t seed, uint64_t stream, double mean, double std, int64_t n, uint16_t* out) {
    const uint64_t key = stream_key(seed, stream);
    const int64_t npairs = (n + 1) / 2;
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < npairs; c += CHUNK) {
        int64_t e = c + CHUNK < npairs ? c + CHUNK : npairs;
        for (int64_t p = c; p < e; ++p) {
            double z0, z1;
            normal_pair(key, p, &z0, &z1);
            out[2 * p] = f32_to_bf16_rne((float)(mean + std * z0));
            if (2 * p + 1 < n) out[2 * p + 1] = f32_to_bf16_rne((float)(mean + std * z1));
        }
    }
}

/* uniform integers in [lo, hi] (inclusive), by multiply-shift on 32 bits */
void synth_uniform_int(uint64_t seed, uint64_t stream, int64_t lo, int64_t hi, int64_t n, int64_t* out) {
    const uint64_t key = stream_key(seed, stream);
    const uint64_t span = (uint64_t)(hi - lo + 1);
    for (int64_t i = 0; i < n; ++i) {
        uint64_t w = splitmix64(key + (uint64_t)i);
        /* 128-bit multiply-high maps w uniformly (to within 2^-64) onto span */
        unsigned __int128 m = (unsigned __int128)w * span;
        out[i] = lo + (int64_t)(uint64_t)(m >> 64);
    }
}

/* uniform doubles in (0, 1] */
void synth_uniform_f64(uint64_t seed, uint64_t stream, int64_t n, double* out) {
    const uint64_t key = stream_key(seed, stream);
    for (int64_t i = 0; i < n; ++i) out[i] = u01(splitmix64(key + (uint64_t)i));
}

/* copy a value-initialised bf16 constant (used for norm gains = 1.0) */
void synth_fill_u16(uint16_t v, int64_t n, uint16_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = v;
}

/* n_bytes bytes of 4-bit codes, two per byte: byte i holds code 2i in its
 * low nibble and code 2i + 1 in its high nibble (the layout of the W4
 * matrices, codes in row order). The codes are those of Gaussian weights
 * under symmetric 4-bit quantization: code = clamp(round(sigma * z) + 8,
 * 0, 15), with z0, z1 of normal pair i for codes 2i and 2i + 1. Every
 * code occurs (0 and 15 through the clamp), and the dequantized values
 * (code - 8) have mean about zero. */
void synth_codes_u4(uint64_t seed, uint64_t stream, double sigma, int64_t n_bytes, uint8_t* out) {
    const uint64_t key = stream_key(seed, stream);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n_bytes; ++i) {
        double z0, z1;
        normal_pair(key, i, &z0, &z1);
        long c0 = lround(sigma * z0) + 8, c1 = lround(sigma * z1) + 8;
        c0 = c0 < 0 ? 0 : c0 > 15 ? 15 : c0;
        c1 = c1 < 0 ? 0 : c1 > 15 ? 15 : c1;
        out[i] = (uint8_t)(c0 | (c1 << 4));
    }
}
