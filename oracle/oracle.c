/*
 * oracle/oracle.c -- the CPU oracle of the block-scaled low-bit MoE layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
 * CPU-baseline leg may load this library.  The GPU library never calls it and
 * shares no code, header, table or constant with it.
 *
 * Plain, slow and meant to be checked by eye: every weight is decoded through
 * an explicit value table that is built here by enumerating the bit fields of
 * each format, and every product and sum is formed in double precision in the
 * order the definitions state.  Parallel loops (OpenMP) only split independent
 * output elements; no sum is reordered.
 *
 * Sources (the four pages, cited by title and section):
 *  - knivesysl README, "formats": 6-bit e2m3 values with a power-of-two scale
 *    per 128 weights; 4-bit values with a scale per 16 (nvfp4); and its
 *    "current benchmark" section, whose numeric gate decodes the same packed
 *    bytes in FP64 -- the model for this file.
 *  - colibri README, "DeepSeek V4": native fp4 experts, fp8-e4m3 with UE8M0
 *    block scales, routed experts plus one shared expert, top-k routing.
 *  - Strata docs/INTEL.md, "The engine itself on Intel": router_top10 and
 *    shared_expert kernels; nextsycl README, "What it does" and "Lessons
 *    learned": SwiGLU experts split as gate | up followed by down.
 * Readings the pages leave open (bit order, tie-break, gate function, shared
 * weight, subnormals, the e4m3 variant) are the plainest ones and are listed
 * with the design notes.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_FMT_E2M1 1        /* e2m1 codes, fp8 e4m3 scale per 16 weights */
#define ORACLE_FMT_E2M3 2        /* e2m3 codes, UE8M0 (power of two) scale per 128 weights */
#define ORACLE_FMT_MXFP4 3       /* e2m1 codes, UE8M0 scale per 32 weights (colibri README, model
                                    notes: Kimi K3's MXFP4 experts) */
#define ORACLE_FMT_INT4_F16 4    /* int4 codes, fp16 scale per 64 weights (colibri README, "Get the
                                    model": the group-scaled gs64 int4 container) */
#define ORACLE_FMT_E2M3_E4M3 5   /* e2m3 codes, fp8 e4m3 scale per 16 weights */

static double T_E2M1[16];
static double T_E2M3[64];
static double T_E4M3[256];
static double T_UE8M0[256];
static double T_INT4[16];
static int tables_ready = 0;

/* A minifloat with one sign bit, ebits exponent bits of bias `bias`, mbits
 * mantissa bits, subnormals at exponent field 0 and no infinities:
 *   e == 0 : (m / 2^mbits) * 2^(1 - bias)
 *   e >  0 : (1 + m / 2^mbits) * 2^(e - bias)                                */
static double minifloat(unsigned code, int ebits, int mbits, int bias) {
    unsigned m = code & ((1u << mbits) - 1u);
    unsigned e = (code >> mbits) & ((1u << ebits) - 1u);
    unsigned s = (code >> (mbits + ebits)) & 1u;
    double mag;
    if (e == 0) mag = ldexp((double)m / (double)(1u << mbits), 1 - bias);
    else        mag = ldexp(1.0 + (double)m / (double)(1u << mbits), (int)e - bias);
    return s ? -mag : mag;
}

static void build_tables(void) {
    if (tables_ready) return;
    for (unsigned c = 0; c < 16; ++c) T_E2M1[c] = minifloat(c, 2, 1, 1);      /* e2m1, bias 1 */
    for (unsigned c = 0; c < 64; ++c) T_E2M3[c] = minifloat(c, 2, 3, 1);      /* e2m3, bias 1 */
    for (unsigned b = 0; b < 256; ++b) {
        /* e4m3 "FN": bias 7, no infinities, exponent and mantissa all ones is NaN */
        if ((b & 0x7F) == 0x7F) T_E4M3[b] = NAN;
        else T_E4M3[b] = minifloat(b, 4, 3, 7);
        /* UE8M0: unsigned, eight exponent bits, bias 127, no mantissa; 0xFF is NaN */
        T_UE8M0[b] = (b == 0xFF) ? NAN : ldexp(1.0, (int)b - 127);
    }
    /* int4: the code read as a two's-complement 4-bit integer (bit 3 weighs -8) */
    for (unsigned c = 0; c < 16; ++c) T_INT4[c] = (double)(c & 7u) - ((c & 8u) ? 8.0 : 0.0);
    tables_ready = 1;
}

/* IEEE 754 binary16 from its bit fields: sign bit 15, five exponent bits of
 * bias 15, ten mantissa bits.  Exponent field 0: subnormal (m / 2^10) * 2^-14;
 * field 31: infinity (m == 0) or NaN. */
static double fp16_value(unsigned h) {
    unsigned s = (h >> 15) & 1u, e = (h >> 10) & 31u, m = h & 1023u;
    double mag;
    if (e == 31) mag = m ? NAN : INFINITY;
    else if (e == 0) mag = ldexp((double)m / 1024.0, -14);
    else mag = ldexp(1.0 + (double)m / 1024.0, (int)e - 15);
    return s ? -mag : mag;
}

double oracle_fp16_value(unsigned h) { return fp16_value(h); }

void oracle_int4_table(double *int4) {
    build_tables();
    memcpy(int4, T_INT4, sizeof T_INT4);
}

int oracle_init(void) { build_tables(); return 0; }

/* Threads of the parallel loops that follow (n <= 0: leave as is); returns
 * the count now in force.  Only splits independent outputs: no result
 * depends on it. */
#ifdef _OPENMP
#include <omp.h>
#endif
int oracle_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
    return omp_get_max_threads();
#else
    (void)n;
    return 1;
#endif
}

void oracle_tables(double *e2m1, double *e2m3, double *e4m3, double *ue8m0) {
    build_tables();
    memcpy(e2m1, T_E2M1, sizeof T_E2M1);
    memcpy(e2m3, T_E2M3, sizeof T_E2M3);
    memcpy(e4m3, T_E4M3, sizeof T_E4M3);
    memcpy(ue8m0, T_UE8M0, sizeof T_UE8M0);
}

/* bf16 is the upper half of an IEEE binary32 */
static double bf16_value(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

double oracle_bf16_value(uint16_t h) { return bf16_value(h); }

/* Formats whose codes are four bits wide (two per byte); the others are six. */
static int four_bit(int fmt) { return fmt == ORACLE_FMT_E2M1 || fmt == ORACLE_FMT_MXFP4 || fmt == ORACLE_FMT_INT4_F16; }

int64_t oracle_code_row_bytes(int fmt, int64_t cols) { return four_bit(fmt) ? cols / 2 : cols * 3 / 4; }

/* Scale bytes per row: one byte per block of 16 (e4m3), 32 or 128 (UE8M0)
 * weights; two bytes (little-endian fp16) per group of 64 for int4. */
int64_t oracle_scale_row_bytes(int fmt, int64_t cols) {
    switch (fmt) {
        case ORACLE_FMT_E2M1: case ORACLE_FMT_E2M3_E4M3: return cols / 16;
        case ORACLE_FMT_E2M3: return cols / 128;
        case ORACLE_FMT_MXFP4: return cols / 32;
        default: return 2 * (cols / 64);
    }
}

/* The code of element j in one packed row. */
static unsigned code_at(int fmt, const uint8_t *row, int64_t j) {
    if (four_bit(fmt)) {
        uint8_t b = row[j >> 1];
        return (j & 1) ? (b >> 4) : (b & 0x0F);          /* low nibble holds the even element */
    }
    /* e2m3: bits 6j .. 6j+5 of the row, bit i of the row being bit (i mod 8) of byte i/8 */
    unsigned c = 0;
    for (int t = 0; t < 6; ++t) {
        int64_t bit = 6 * j + t;
        c |= (unsigned)((row[bit >> 3] >> (bit & 7)) & 1) << t;
    }
    return c;
}

/* W[j] of one row: the code's value times its block's scale (exact in double). */
static double weight_at(int fmt, const uint8_t *crow, const uint8_t *srow, int64_t j) {
    const unsigned c = code_at(fmt, crow, j);
    switch (fmt) {
        case ORACLE_FMT_E2M1: return T_E2M1[c] * T_E4M3[srow[j / 16]];
        case ORACLE_FMT_E2M3: return T_E2M3[c] * T_UE8M0[srow[j / 128]];
        case ORACLE_FMT_MXFP4: return T_E2M1[c] * T_UE8M0[srow[j / 32]];
        case ORACLE_FMT_E2M3_E4M3: return T_E2M3[c] * T_E4M3[srow[j / 16]];
        default: {   /* int4: the group's fp16 scale, low byte first */
            const uint8_t *g = srow + 2 * (j / 64);
            return T_INT4[c] * fp16_value((unsigned)g[0] | ((unsigned)g[1] << 8));
        }
    }
}

/* Decode a whole matrix [rows][cols] to double. */
void oracle_decode(int fmt, int64_t rows, int64_t cols, const uint8_t *codes, const uint8_t *scales, double *out) {
    build_tables();
    const int64_t cb = oracle_code_row_bytes(fmt, cols), sb = oracle_scale_row_bytes(fmt, cols);
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t j = 0; j < cols; ++j)
            out[r * cols + j] = weight_at(fmt, codes + r * cb, scales + r * sb, j);
}

/* One dot product: row r of W with a bf16 vector, summed j = 0 .. cols-1. */
static double row_dot_bf16(int fmt, int64_t cols, const uint8_t *crow, const uint8_t *srow, const uint16_t *x) {
    double acc = 0.0;
    for (int64_t j = 0; j < cols; ++j) acc += weight_at(fmt, crow, srow, j) * bf16_value(x[j]);
    return acc;
}

static double row_dot_f64(int fmt, int64_t cols, const uint8_t *crow, const uint8_t *srow, const double *x) {
    double acc = 0.0;
    for (int64_t j = 0; j < cols; ++j) acc += weight_at(fmt, crow, srow, j) * x[j];
    return acc;
}

/* Dense GEMV: y[b][i] = sum_j W[row_i][j] * x[b][j] for the rows in row_list
 * (all rows, in order, when row_list is NULL; n_rows is then `rows`). */
void oracle_gemv(int fmt, int64_t rows, int64_t cols, const uint8_t *codes, const uint8_t *scales,
                 const uint16_t *x, int64_t B, const int64_t *row_list, int64_t n_rows, double *y) {
    build_tables();
    const int64_t cb = oracle_code_row_bytes(fmt, cols), sb = oracle_scale_row_bytes(fmt, cols);
    if (!row_list) n_rows = rows;
    #pragma omp parallel for schedule(dynamic, 16)
    for (int64_t i = 0; i < n_rows; ++i) {
        int64_t r = row_list ? row_list[i] : i;
        for (int64_t b = 0; b < B; ++b)
            y[b * n_rows + i] = row_dot_bf16(fmt, cols, codes + r * cb, scales + r * sb, x + b * cols);
    }
}

/* Ordering used by routing: a ranks before b when its logit is larger; equal
 * logits (+0 and -0 are equal) rank by the lower expert index; NaN ranks below
 * every number. */
static int ranks_before(const float *l, int32_t a, int32_t b) {
    float la = l[a], lb = l[b];
    int na = isnan(la), nb = isnan(lb);
    if (na || nb) {
        if (na && nb) return a < b;
        return nb;                   /* the non-NaN one ranks first */
    }
    if (la > lb) return 1;
    if (la < lb) return 0;
    return a < b;
}

/* Top-k routing for T tokens: idx[t][r] are the k best experts in rank order,
 * w[t][r] = exp(l_r - l_0) / sum_s exp(l_s - l_0) over the k selected logits
 * (softmax over all E logits renormalised over the k kept equals this). */
int oracle_route(const float *logits, int64_t T, int64_t E, int64_t k, int32_t *idx, double *w) {
    if (k < 1 || k > E) return -1;
    char *taken = (char *)malloc((size_t)E);
    if (!taken) return -2;
    for (int64_t t = 0; t < T; ++t) {
        const float *l = logits + t * E;
        memset(taken, 0, (size_t)E);
        for (int64_t r = 0; r < k; ++r) {            /* selection: k passes for the best remaining */
            int32_t best = -1;
            for (int32_t e = 0; e < (int32_t)E; ++e) {
                if (taken[e]) continue;
                if (best < 0 || ranks_before(l, e, best)) best = e;
            }
            taken[best] = 1;
            idx[t * k + r] = best;
        }
        double l0 = (double)l[idx[t * k]], z = 0.0;
        for (int64_t r = 0; r < k; ++r) z += exp((double)l[idx[t * k + r]] - l0);
        for (int64_t r = 0; r < k; ++r) w[t * k + r] = exp((double)l[idx[t * k + r]] - l0) / z;
    }
    free(taken);
    return 0;
}

double oracle_silu(double z) { return z / (1.0 + exp(-z)); }

/* One SwiGLU expert on one token x (bf16, length H):
 *   g_i = Wg[i].x,  u_i = Wu[i].x   (rows 0..I-1 of w13 are gate, I..2I-1 up)
 *   h_i = silu(g_i) * u_i
 *   y_o = Wd[o].h                    for o in out_rows (all H rows if NULL)
 * h_out (length I) receives h when not NULL. */
void oracle_ffn(int fmt, int64_t H, int64_t I,
                const uint8_t *w13c, const uint8_t *w13s, const uint8_t *w2c, const uint8_t *w2s,
                const uint16_t *x, const int64_t *out_rows, int64_t n_out, double *h_out, double *y) {
    build_tables();
    const int64_t cbH = oracle_code_row_bytes(fmt, H), sbH = oracle_scale_row_bytes(fmt, H);
    const int64_t cbI = oracle_code_row_bytes(fmt, I), sbI = oracle_scale_row_bytes(fmt, I);
    double *h = (double *)malloc((size_t)I * sizeof(double));
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < I; ++i) {
        double g = row_dot_bf16(fmt, H, w13c + i * cbH, w13s + i * sbH, x);
        double u = row_dot_bf16(fmt, H, w13c + (I + i) * cbH, w13s + (I + i) * sbH, x);
        h[i] = oracle_silu(g) * u;
    }
    if (h_out) memcpy(h_out, h, (size_t)I * sizeof(double));
    if (!out_rows) n_out = H;
    #pragma omp parallel for schedule(static)
    for (int64_t q = 0; q < n_out; ++q) {
        int64_t o = out_rows ? out_rows[q] : q;
        y[q] = row_dot_f64(fmt, I, w2c + o * cbI, w2s + o * sbI, h);
    }
    free(h);
}

/* The layer for T tokens:
 *   out[t][o] = sum_{r=0..k-1} w[t][r] * FFN_{idx[t][r]}(x_t)[o]  +  FFN_shared(x_t)[o]
 * summed in that order.  Expert weights are passed as arrays of E pointers
 * (entries of experts no token selects may be NULL); the shared expert is
 * present when shared_inter > 0 and enters with weight 1.
 * Returns 0, or -3 when a selected expert's pointers are NULL. */
int oracle_layer(int fmt, int64_t T, int64_t H, int64_t I, int64_t E, int64_t k,
                 const uint8_t *const *w13c, const uint8_t *const *w13s,
                 const uint8_t *const *w2c, const uint8_t *const *w2s,
                 int64_t shared_inter, const uint8_t *sh13c, const uint8_t *sh13s,
                 const uint8_t *sh2c, const uint8_t *sh2s,
                 const uint16_t *x, const float *logits,
                 const int64_t *out_rows, int64_t n_out,
                 int32_t *idx, double *w, double *out) {
    build_tables();
    if (!out_rows) n_out = H;
    int rc = oracle_route(logits, T, E, k, idx, w);
    if (rc) return rc;
    double *y = (double *)malloc((size_t)n_out * sizeof(double));
    for (int64_t t = 0; t < T; ++t) {
        double *o = out + t * n_out;
        for (int64_t q = 0; q < n_out; ++q) o[q] = 0.0;
        for (int64_t r = 0; r < k; ++r) {
            int32_t e = idx[t * k + r];
            if (!w13c[e] || !w13s[e] || !w2c[e] || !w2s[e]) { free(y); return -3; }
            oracle_ffn(fmt, H, I, w13c[e], w13s[e], w2c[e], w2s[e], x + t * H, out_rows, n_out, NULL, y);
            for (int64_t q = 0; q < n_out; ++q) o[q] += w[t * k + r] * y[q];
        }
        if (shared_inter > 0) {
            oracle_ffn(fmt, H, shared_inter, sh13c, sh13s, sh2c, sh2s, x + t * H, out_rows, n_out, NULL, y);
            for (int64_t q = 0; q < n_out; ++q) o[q] += y[q];
        }
    }
    free(y);
    return 0;
}

/* The steps either side of the MoE layer (the whole MoE block):
 *   RMSNorm in front of it (nextsycl README, dense 27B engine: the norm that
 *   emits the next kernel's input; knivesysl README, "how it works": RMS fused
 *   into the activation quantisation);
 *   the router scores that routing ranks (Strata docs/INTEL.md, "Decode
 *   round 2": scores followed by top-k);
 *   the residual add after it.  */

/* y[t][i] = x[t][i] * g[i] / sqrt(eps + (1/H) * sum_j x[t][j]^2), x and g bf16. */
void oracle_rmsnorm(int64_t T, int64_t H, const uint16_t *x, const uint16_t *g, double eps, double *y) {
    for (int64_t t = 0; t < T; ++t) {
        const uint16_t *xt = x + t * H;
        double ss = 0.0;
        for (int64_t j = 0; j < H; ++j) ss += bf16_value(xt[j]) * bf16_value(xt[j]);
        const double r = 1.0 / sqrt(ss / (double)H + eps);
        for (int64_t i = 0; i < H; ++i) y[t * H + i] = bf16_value(xt[i]) * bf16_value(g[i]) * r;
    }
}

/* logits[t][e] = sum_j Wr[e][j] * x[t][j]: router weights bf16 [E][H], x bf16 [T][H]. */
void oracle_router_logits(int64_t T, int64_t H, int64_t E, const uint16_t *x, const uint16_t *wr, double *logits) {
    #pragma omp parallel for schedule(static)
    for (int64_t e = 0; e < E; ++e)
        for (int64_t t = 0; t < T; ++t) {
            double acc = 0.0;
            for (int64_t j = 0; j < H; ++j) acc += bf16_value(wr[e * H + j]) * bf16_value(x[t * H + j]);
            logits[t * E + e] = acc;
        }
}

/* out[t][i] = r[t][i] + y[t][i]: the residual stream r (bf16) plus the block's output. */
void oracle_residual_add(int64_t n, const uint16_t *r, const double *y, double *out) {
    for (int64_t i = 0; i < n; ++i) out[i] = bf16_value(r[i]) + y[i];
}

/* ---- Activation quantisation for the scaled matrix cores (the pages' fp6
 * path with e4m3 activations: knivesysl README, "formats" and "key flags";
 * amax scaling as in Strata docs/INTEL.md, "The engine itself on Intel",
 * whose activation quantiser is byte-exact to its reference).  MX element
 * format e4m3 with a UE8M0 scale per block of 32 consecutive elements of a
 * row, by the OCP MX rule:
 *   amax = max |x| over the block;
 *   scale exponent X = floor(log2(amax)) - 8 (8: the largest binade of e4m3,
 *   whose largest value is 448 = 1.75 * 2^8), clamped to [-127, 127]; a block
 *   of zeros takes X = -127;
 *   each element: x / 2^X rounded to the nearest e4m3 value, ties to the even
 *   code, magnitudes above 448 saturated to 448; the sign kept (-0 too).
 * The dequantised element is value(code) * 2^X. */

/* The e4m3 code nearest to v (ties to the even code), saturating at 448. */
static uint8_t e4m3_nearest(double v) {
    const uint8_t s = signbit(v) ? 0x80 : 0x00;
    const double a = fabs(v);
    unsigned best = 0;
    double bd = INFINITY;
    for (unsigned c = 0; c < 0x7F; ++c) {           /* the 127 finite non-negative codes, in value order */
        const double d = fabs(T_E4M3[c] - a);
        if (d < bd || (d == bd && (c & 1u) == 0)) { bd = d; best = c; }
    }
    return (uint8_t)(s | best);
}

void oracle_quantize_mx_e4m3(int64_t T, int64_t H, const uint16_t *x, uint8_t *codes, uint8_t *scales) {
    build_tables();
    for (int64_t t = 0; t < T; ++t)
        for (int64_t b = 0; b < H / 32; ++b) {
            const uint16_t *xb = x + t * H + 32 * b;
            double amax = 0.0;
            for (int j = 0; j < 32; ++j) amax = fmax(amax, fabs(bf16_value(xb[j])));
            int X = -127;
            if (amax > 0.0) {
                int e;
                frexp(amax, &e);                     /* amax = f * 2^e, f in [0.5, 1): floor(log2 amax) = e - 1 */
                X = (e - 1) - 8;
                if (X < -127) X = -127;
                if (X > 127) X = 127;
            }
            scales[t * (H / 32) + b] = (uint8_t)(X + 127);
            for (int j = 0; j < 32; ++j) codes[t * H + 32 * b + j] = e4m3_nearest(ldexp(bf16_value(xb[j]), -X));
        }
}

/* Round a double to bfloat16, once, to nearest with ties to even.  Rounding
 * works on the significand scaled to eight bits (normal range) or on the
 * fixed unit 2^-133 (subnormal range). */
uint16_t oracle_bf16_round(double v) {
    if (isnan(v)) return 0x7FC0;
    uint16_t s = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (a == 0.0) return s;
    if (isinf(a)) return (uint16_t)(s | 0x7F80);
    if (a < ldexp(1.0, -126)) return (uint16_t)(s | (uint16_t)nearbyint(ldexp(a, 133)));
    int e;
    double f = frexp(a, &e);
    double q = nearbyint(ldexp(f, 8));
    if (q == 256.0) { q = 128.0; ++e; }
    int E8 = e - 1 + 127;
    if (E8 >= 255) return (uint16_t)(s | 0x7F80);
    return (uint16_t)(s | (E8 << 7) | ((int)q - 128));
}

void oracle_bf16_round_array(const double *v, int64_t n, uint16_t *out) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_bf16_round(v[i]);
}
