/*
 * synth/gen.c -- seeded, counter-based generator of synthetic inputs.
 *
 * This module produces the random bytes and numbers that both the GPU library
 * and the CPU oracle consume.  It holds none of the method's arithmetic: it
 * never decodes a weight, never multiplies a matrix and never routes a token.
 * The only format knowledge here is how to *draw* a scale byte whose value
 * follows a requested distribution (an encoder), which the decoders on both
 * sides never use.
 *
 * Counter-based SplitMix64 (Steele, Lea & Flood, "Fast splittable pseudorandom
 * number generators", OOPSLA 2014): word(seed, stream, c) is the SplitMix64
 * output function applied to key(seed, stream) + (c + 1) * GAMMA, where the key
 * is itself a mixed function of (seed, stream).  Any element of any tensor can
 * therefore be produced alone, in any order, by any number of threads.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

static inline uint64_t stream_key(uint64_t seed, uint64_t stream) {
    return mix64(mix64(seed * GAMMA + 0x632BE59BD9B4E019ULL) ^ (stream * 0xD1B54A32D192ED03ULL + GAMMA));
}

static inline uint64_t word_at(uint64_t key, uint64_t c) { return mix64(key + (c + 1) * GAMMA); }

/* 53-bit uniform in [0, 1) */
static inline double unit53(uint64_t w) { return (double)(w >> 11) * (1.0 / 9007199254740992.0); }

uint64_t synth_word(uint64_t seed, uint64_t stream, uint64_t c) { return word_at(stream_key(seed, stream), c); }

/* Uniform random bytes: byte j of the stream is byte (j & 7) of word j >> 3. */
void synth_bytes(uint64_t seed, uint64_t stream, uint64_t offset, uint64_t n, uint8_t *out) {
    const uint64_t key = stream_key(seed, stream);
    #pragma omp parallel for schedule(static) if (n > (1u << 20))
    for (int64_t i = 0; i < (int64_t)n; ++i) {
        uint64_t j = offset + (uint64_t)i;
        out[i] = (uint8_t)(word_at(key, j >> 3) >> (8 * (j & 7)));
    }
}

/* Round a positive finite double to the nearest fp8 E4M3 (FN variant: bias 7,
 * three mantissa bits, subnormals at exponent field 0), ties to even.
 * Values beyond the largest finite (448) saturate to it.  Returns the byte. */
static uint8_t e4m3_encode_pos(double v) {
    if (!(v > 0)) return 0;
    if (v >= 448.0) return 0x7E;
    if (v < ldexp(1.0, -6)) {                 /* subnormal: unit 2^-9 */
        double r = nearbyint(ldexp(v, 9));    /* 0..8; 8 means 2^-6, the smallest normal */
        return (uint8_t)r;                    /* code 8 == exponent field 1, mantissa 0 */
    }
    int e;
    double f = frexp(v, &e);                  /* v = f * 2^e, f in [0.5, 1) */
    double r = nearbyint(ldexp(f, 4));        /* 4 significant bits: 8..16 */
    if (r == 16.0) { r = 8.0; e += 1; }
    int ef = (e - 1) + 7;
    if (ef > 15 || (ef == 15 && r - 8.0 >= 7.0)) return 0x7E;
    return (uint8_t)((ef << 3) | (int)(r - 8.0));
}

/* Scale bytes whose values are log-uniform: 2^u, u ~ U[lo, hi), rounded to E4M3. */
void synth_e4m3_loguniform(uint64_t seed, uint64_t stream, uint64_t offset, uint64_t n,
                           double lo, double hi, uint8_t *out) {
    const uint64_t key = stream_key(seed, stream);
    #pragma omp parallel for schedule(static) if (n > (1u << 18))
    for (int64_t i = 0; i < (int64_t)n; ++i) {
        double u = lo + (hi - lo) * unit53(word_at(key, offset + (uint64_t)i));
        out[i] = e4m3_encode_pos(exp2(u));
    }
}

/* UE8M0 scale bytes for 2^e with the integer exponent e uniform over [lo, hi]. */
void synth_ue8m0_uniform(uint64_t seed, uint64_t stream, uint64_t offset, uint64_t n,
                         int lo, int hi, uint8_t *out) {
    const uint64_t key = stream_key(seed, stream);
    const uint64_t span = (uint64_t)(hi - lo + 1);
    #pragma omp parallel for schedule(static) if (n > (1u << 18))
    for (int64_t i = 0; i < (int64_t)n; ++i) {
        uint64_t w = word_at(key, offset + (uint64_t)i);
        uint64_t pick = ((w >> 32) * span) >> 32;      /* multiply-shift: uniform over span */
        out[i] = (uint8_t)(127 + lo + (int)pick);
    }
}

/* Round a double in fp16's positive normal range [2^-14, 65504] to the nearest
 * IEEE binary16 (ten mantissa bits), ties to even.  Returns the bit pattern. */
static uint16_t fp16_encode_pos_normal(double v) {
    int e;
    double f = frexp(v, &e);                  /* v = f * 2^e, f in [0.5, 1) */
    double r = nearbyint(ldexp(f, 11));       /* 11 significant bits: 1024..2048 */
    if (r == 2048.0) { r = 1024.0; e += 1; }
    return (uint16_t)(((e - 1 + 15) << 10) | (int)(r - 1024.0));
}

/* fp16 group scales 2^u, u ~ U[lo, hi), rounded to binary16, stored as two
 * bytes each, low byte first (lo and hi keep the values normal). */
void synth_fp16_loguniform(uint64_t seed, uint64_t stream, uint64_t offset, uint64_t n,
                           double lo, double hi, uint8_t *out) {
    const uint64_t key = stream_key(seed, stream);
    #pragma omp parallel for schedule(static) if (n > (1u << 18))
    for (int64_t i = 0; i < (int64_t)n; ++i) {
        double u = lo + (hi - lo) * unit53(word_at(key, offset + (uint64_t)i));
        uint16_t h = fp16_encode_pos_normal(exp2(u));
        out[2 * i] = (uint8_t)(h & 0xFF);
        out[2 * i + 1] = (uint8_t)(h >> 8);
    }
}

uint16_t synth_fp16_encode(double v) { return fp16_encode_pos_normal(v); }

/* Standard normal by Box-Muller (cosine branch), one normal per counter, from
 * two 53-bit uniforms taken from words 2c and 2c+1. */
static inline double normal_at(uint64_t key, uint64_t c) {
    double u1 = unit53(word_at(key, 2 * c)) + (1.0 / 9007199254740992.0);   /* (0, 1] */
    double u2 = unit53(word_at(key, 2 * c + 1));
    return sqrt(-2.0 * log(u1)) * cos(6.283185307179586476925286766559 * u2);
}

/* Round a double to bfloat16 with one round-to-nearest-even (no detour through
 * float, which would round twice). */
static uint16_t bf16_from_double(double v) {
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (isnan(v)) return 0x7FC0;
    if (a == 0) return sign;
    if (a < ldexp(1.0, -126)) {                          /* subnormal: unit 2^-133 */
        double r = nearbyint(ldexp(a, 133));              /* 0..128; 128 -> smallest normal */
        return (uint16_t)(sign | (uint16_t)r);
    }
    int e;
    double f = frexp(a, &e);                               /* a = f * 2^e */
    double r = nearbyint(ldexp(f, 8));                     /* 8 significant bits: 128..256 */
    if (r == 256.0) { r = 128.0; e += 1; }
    int ef = (e - 1) + 127;
    if (ef >= 255) return (uint16_t)(sign | 0x7F80);       /* overflow to infinity */
    return (uint16_t)(sign | (ef << 7) | ((int)r - 128));
}

void synth_normal_bf16(uint64_t seed, uint64_t stream, uint64_t offset, uint64_t n,
                       double sigma, uint16_t *out) {
    const uint64_t key = stream_key(seed, stream);
    #pragma omp parallel for schedule(static) if (n > (1u << 18))
    for (int64_t i = 0; i < (int64_t)n; ++i)
        out[i] = bf16_from_double(sigma * normal_at(key, offset + (uint64_t)i));
}

/* bf16 of mean + sigma * N(0,1), rounded once (gains around a mean). */
void synth_normal_bf16_mean(uint64_t seed, uint64_t stream, uint64_t offset, uint64_t n, double mean,
                            double sigma, uint16_t *out) {
    const uint64_t key = stream_key(seed, stream);
    #pragma omp parallel for schedule(static) if (n > (1u << 18))
    for (int64_t i = 0; i < (int64_t)n; ++i) out[i] = bf16_from_double(mean + sigma * normal_at(key, offset + (uint64_t)i));
}

void synth_normal_f32(uint64_t seed, uint64_t stream, uint64_t offset, uint64_t n,
                      double sigma, float *out) {
    const uint64_t key = stream_key(seed, stream);
    #pragma omp parallel for schedule(static) if (n > (1u << 18))
    for (int64_t i = 0; i < (int64_t)n; ++i)
        out[i] = (float)(sigma * normal_at(key, offset + (uint64_t)i));  /* one RNE */
}

/* Exposed for the generator's own tests. */
uint16_t synth_bf16_from_double(double v) { return bf16_from_double(v); }
uint8_t synth_e4m3_encode(double v) { return e4m3_encode_pos(v); }
