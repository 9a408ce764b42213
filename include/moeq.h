/*
 * moeq.h -- C ABI of the block-scaled low-bit MoE decode library (MI355X, gfx950).
 *
 * The operation: a mixture-of-experts FFN layer whose expert weights are stored
 * as block-scaled low-bit codes.  For each token the router logits pick the k
 * best experts (top-k), their gate weights are the softmax of the k picked
 * logits, each picked expert runs a SwiGLU FFN (gate | up projections, SiLU of
 * the gate times the up, down projection) and the results are summed with
 * those weights, plus an always-on shared expert with weight 1.
 *
 * Where each piece is stated (the pages, by title and section):
 *  - weight formats: knivesysl README, "formats" (six-bit e2m3 values with a
 *    power-of-two scale per 128 weights; four-bit nvfp4 values with a scale per
 *    16) and "key flags" (the 4-bit e2m1 weight tier); colibri README,
 *    "DeepSeek V4" (UE8M0 block scales, fp8-e4m3).
 *  - routing and the shared expert: Strata docs/INTEL.md, "The engine itself on
 *    Intel" (the router_top10 and shared_expert kernels); colibri README,
 *    "DeepSeek V4" (routed experts plus one shared expert, top-k).
 *  - the expert FFN split as gate | up then down: nextsycl README, "What it
 *    does" and "Lessons learned".
 *  - batched decode rows that must each equal their own one-row pass: nextsycl
 *    README, "What it does" (several requests at once) and "Lessons learned".
 *  - a native library behind a C ABI, loaded from Python: knivesysl README,
 *    introduction; errors that name the failing operation: its "current
 *    benchmark" section.
 *
 * Data layout (all row-major, every row contiguous; codes and scales planar):
 *   MOE_FMT_E2M1_E4M3_B16   codes  [rows][cols/2]   element j in byte j>>1,
 *                                                    low nibble = even element
 *                           scales [rows][cols/16]  fp8 e4m3 (OCP "FN": bias 7,
 *                                                    no Inf, 0x7F/0xFF = NaN)
 *   MOE_FMT_E2M3_UE8M0_B128 codes  [rows][3*cols/4] element j in bits
 *                                                    [6j, 6j+6) of the row read
 *                                                    as a little-endian bit string
 *                           scales [rows][cols/128] UE8M0: value 2^(b-127)
 *   MOE_FMT_E2M1_UE8M0_B32  codes  as format 1
 *                           scales [rows][cols/32]  UE8M0
 *   MOE_FMT_INT4_F16_B64    codes  as format 1, each nibble a two's-complement
 *                                                    integer -8..7
 *                           scales [rows][cols/64]  IEEE binary16, two bytes
 *                                                    each, low byte first
 *   MOE_FMT_E2M3_E4M3_B16   codes  as format 2
 *                           scales [rows][cols/16]  fp8 e4m3 as format 1
 *   Weight W[r][j] = value(code) * value(scale[r][j / block]); e2m1 and e2m3
 *   have one sign bit, two exponent bits of bias 1 and 1 or 3 mantissa bits,
 *   with subnormals at exponent field 0 and no Inf/NaN codes.
 *   An expert's w13 is [2*inter][hidden]: rows 0..inter-1 are the gate
 *   projection, rows inter..2*inter-1 the up projection.  w2 is
 *   [hidden][inter].  Routed experts are stacked: expert e's w13 codes begin
 *   at w13_codes + e * 2*inter * code_row_bytes(hidden), and so on.
 *   Activations x are bf16 [T][hidden]; logits fp32 [T][n_experts]; outputs
 *   bf16 (or fp32 with MOE_OUT_F32) [T][hidden].
 *
 * Conventions for every call:
 *  - Pointers to data are DEVICE pointers (hipMalloc'd or torch CUDA tensors)
 *    unless stated otherwise; descriptor structs are host memory, read only
 *    during the call.  The caller owns every buffer.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *    on it and the call returns; inputs must stay alive and unchanged until the
 *    stream has passed the call.  No call allocates, frees or synchronises.
 *  - Validation happens before anything is enqueued: on a negative return
 *    nothing was enqueued, outputs are untouched, and moe_last_error() returns
 *    text naming the argument and the rule it broke (thread-local).
 *  - Device pointers must be 16-byte aligned; workspaces 256-byte aligned.
 *    Code and scale arrays are read in 16-byte pieces: when an array's length
 *    is not a multiple of 16, the bytes up to the end of its last 16-byte
 *    granule may be read (and ignored); they never lie outside that granule.
 *  - Arithmetic: weights are decoded exactly, products and sums are formed in
 *    fp32, the SiLU and the softmax in fp32, and the output is rounded to bf16
 *    once (round to nearest even).  Routing compares the raw fp32 logits and
 *    is bit-exact: larger logit first, equal logits (+0 == -0) by lower expert
 *    index, NaN below every number.  A token's result does not depend on which
 *    other tokens share the call.
 *  - The library keeps no state between calls except facts about each device
 *    that a launch needs (CU count, occupancy), looked up once and cached on
 *    the host behind a lock.  Calls may come from several threads; calls on
 *    different streams need different workspaces.
 */
#ifndef MOEQ_H
#define MOEQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
enum {
    MOE_OK = 0,
    MOE_EINVAL = -1,        /* an argument breaks a documented rule */
    MOE_EUNSUPPORTED = -2,  /* valid, but outside what this library implements */
    MOE_EWORKSPACE = -3,    /* workspace missing, misaligned or too small */
    MOE_EHIP = -4,          /* a HIP runtime call failed (text holds its error) */
    MOE_EKERNEL = -5        /* a kernel's bounded wait expired (moe_workspace_status) */
};

/* Weight formats.  1 and 2 are the formats of knivesysl README, "formats";
 * 3 and 4 the expert containers of colibri README's model notes (MXFP4
 * experts; the group-scaled "gs64" int4 container of "Get the model"); 5 pairs
 * the six-bit elements with the e4m3 scale per 16. */
enum {
    MOE_FMT_E2M1_E4M3_B16 = 1,    /* 4-bit e2m1, one fp8-e4m3 scale per 16 weights */
    MOE_FMT_E2M3_UE8M0_B128 = 2,  /* 6-bit e2m3, one UE8M0 (power-of-two) scale per 128 */
    MOE_FMT_E2M1_UE8M0_B32 = 3,   /* MXFP4: 4-bit e2m1, one UE8M0 scale per 32 */
    MOE_FMT_INT4_F16_B64 = 4,     /* 4-bit two's-complement integers, one fp16 scale per 64 */
    MOE_FMT_E2M3_E4M3_B16 = 5     /* 6-bit e2m3, one fp8-e4m3 scale per 16 */
};

/* Flags. */
enum {
    MOE_OUT_F32 = 1,        /* write the output as fp32 (the value before bf16 rounding) */
    MOE_ACT_MXFP8 = 1 << 27,    /* quantise the activations entering gate | up to MX e4m3 with a
                                   UE8M0 scale per 32 (moe_quantize_mx_e4m3) and use the quantised
                                   values: with MX weights (formats 2 and 3) the many-token path
                                   then runs gate | up on the scaled low-precision matrix cores;
                                   every other path runs on the dequantised values, which bf16
                                   holds exactly for activations in its normal range */
    MOE_DECODER_LUT = 1 << 28,  /* decode codes through byte-indexed tables in LDS */
    MOE_DECODER_HW = 1 << 29,   /* decode codes with gfx950's fp4/fp6 -> bf16 conversions
                                   (both decoders are exact and give identical results; with
                                   neither flag the library default is used: the hardware
                                   decoder, unless the environment sets MOEQ_DECODER=lut) */
    MOE_DEBUG_SPIN_LIMIT = 1 << 30  /* test hook: inter-workgroup waits give up almost at once,
                                       so the MOE_EKERNEL path can be exercised; output invalid */
};

/* Limits. */
#define MOE_MAX_EXPERTS 1024
#define MOE_MAX_TOPK 32
#define MOE_MAX_TOKENS 65536
#define MOE_MAX_GEMV_BATCH 8
#define MOE_MAX_DIM 32768        /* hidden, inter, rows and cols */

/* A block-scaled matrix [rows][cols]; y = W x reduces over cols.
 * cols must be a multiple of 32 (formats 1 and 3), 64 (4 and 5) or 128 (2). */
typedef struct moe_qmat {
    int32_t fmt;
    int32_t rows;
    int32_t cols;
    int32_t reserved;        /* must be 0 */
    const void *codes;       /* device, rows * code_row_bytes(cols) bytes */
    const void *scales;      /* device, rows * scale_row_bytes(cols) bytes */
} moe_qmat;

/* One MoE layer.  hidden and inter (and shared_inter when nonzero) must be
 * multiples of 32 (formats 1 and 3), 64 (4 and 5) or 128 (2). */
typedef struct moe_layer {
    int32_t fmt;
    int32_t hidden;          /* H */
    int32_t inter;           /* I of every routed expert */
    int32_t n_experts;       /* E, 1..MOE_MAX_EXPERTS */
    int32_t top_k;           /* k, 1..min(E, MOE_MAX_TOPK) */
    int32_t shared_inter;    /* I of the shared expert; 0 = no shared expert */
    const void *w13_codes, *w13_scales;   /* [E][2I][H] */
    const void *w2_codes, *w2_scales;     /* [E][H][I]  */
    const void *sh13_codes, *sh13_scales; /* [2*shared_inter][H] (NULL if none) */
    const void *sh2_codes, *sh2_scales;   /* [H][shared_inter]   (NULL if none) */
} moe_layer;

/* Top-k routing (the router_top10 step of Strata docs/INTEL.md, "The engine
 * itself on Intel", for any k).
 *   logits: device fp32 [T][E];  idx: device int32 [T][k];  w: device fp32 [T][k]
 * idx[t] holds the k selected experts in rank order; w[t][r] =
 * exp(l_r - l_0) / sum_s exp(l_s - l_0) over the selected logits, so the k
 * weights sum to 1.  Limits: 1 <= T <= MOE_MAX_TOKENS, 1 <= E <=
 * MOE_MAX_EXPERTS, 1 <= k <= min(E, MOE_MAX_TOPK). */
int moe_route_topk(const float *logits, int T, int E, int k, int32_t *idx, float *w, void *stream);

/* Bytes of workspace moe_layer_decode / moe_expert_ffn_q need for T tokens,
 * or 0 when L or T breaks a rule (moe_last_error() then says which).  The
 * workspace holds what the pages' engines keep between their expert kernels
 * (Strata docs/INTEL.md, "The engine itself on Intel": the grouped work list,
 * the gate | up results and the per-expert partial outputs before the
 * combine) plus a small header of counters.  It must be zeroed once after
 * allocation.  The header keeps a call counter that only grows (it tags the
 * values exchanged between workgroups, so a value left by an earlier call is
 * never taken for the current one) and an error word; every other counter is
 * back at zero when a call's kernels end.  One workspace per stream. */
size_t moe_layer_workspace_bytes(const moe_layer *L, int T);

/* One expert's SwiGLU FFN on M rows of x (nextsycl README, "What it does":
 * gate | up, then down).
 *   expert: 0..E-1 for a routed expert, -1 for the shared expert
 *   x: device bf16 [M][H];  y: device [M][H], bf16 or fp32 (MOE_OUT_F32)
 *   ws: device workspace of at least moe_layer_workspace_bytes(L, M). */
int moe_expert_ffn_q(const moe_layer *L, int expert, const void *x, int M, void *y, int flags,
                     void *ws, size_t ws_bytes, void *stream);

/* The whole layer for T tokens (Strata docs/INTEL.md, "The engine itself on
 * Intel": router_top10, the grouped expert kernels and the shared_expert
 * kernel of one MoE layer; colibri README, "DeepSeek V4": routed experts plus
 * one shared expert, top-k): route, group the (token, expert) pairs by
 * expert, run every selected expert once over its tokens, and combine
 *   out[t] = sum_{r<k} w[t][r] * FFN_{idx[t][r]}(x_t) + FFN_shared(x_t)
 * in that order.  idx_out (int32 [T][k]) and w_out (fp32 [T][k]) receive the
 * routing when not NULL.  T <= 16 runs as one kernel launch (decode); larger
 * T runs the grouped-GEMM prefill path (bf16 matrix cores on weights
 * dequantised exactly in registers; with MX activations and MX weights, the
 * scaled fp8 x fp6/fp4 matrix cores on the codes as stored). */
int moe_layer_decode(const moe_layer *L, const void *x, const float *logits, int T, void *out,
                     int32_t *idx_out, float *w_out, int flags, void *ws, size_t ws_bytes,
                     void *stream);

/* moe_layer_decode for callers that cannot allocate (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * kernels and results as moe_layer_decode, with a workspace the library owns
 * instead of the caller's.  That workspace is one static device array of
 * MOE_NOALLOC_WORKSPACE_BYTES per GPU, held from the library's load until the
 * process ends; the call allocates nothing.  Limits: 1 <= T <= 16 (the decode
 * kernels) and moe_layer_workspace_bytes(L, T) <= MOE_NOALLOC_WORKSPACE_BYTES,
 * else MOE_EINVAL / MOE_EWORKSPACE.  The first call on a device clears the
 * array (a fill kernel on `stream`) and must not be made under graph capture
 * (MOE_EHIP names the reason); later calls may be captured.  Every call on a
 * GPU shares its array, which keeps the previous call's contents: calls that
 * overlap on one GPU (other streams, other threads) race and must be
 * serialised by the caller.  An expired in-kernel wait leaves the output
 * invalid and is not reported here (moe_workspace_status needs a caller
 * workspace). */
#define MOE_NOALLOC_WORKSPACE_BYTES ((size_t)64 << 20)
int moe_layer_decode_noalloc(const moe_layer *L, const void *x, const float *logits, int T, void *out,
                             int32_t *idx_out, float *w_out, int flags, void *stream);

/* ---- The steps either side of the layer: the whole MoE block ----
 * RMSNorm in front of the experts (nextsycl README, dense 27B engine: a norm
 * that emits the next kernel's input; knivesysl README, "how it works": RMS
 * fused into the quantisation), the router scores and their top-k as one
 * launch (Strata docs/INTEL.md, "Decode round 2": scores + top-k fused to cut
 * graph nodes), and the residual add after the layer.
 *
 * RMSNorm:  y[t][i] = x[t][i] * gamma[i] / sqrt(mean_j x[t][j]^2 + eps), in
 * fp32 (sum of squares in a fixed order), one rounding to bf16 (or fp32 with
 * MOE_OUT_F32).  x: device bf16 [T][H]; gamma: device bf16 [H]; y: [T][H].
 * 1 <= T <= MOE_MAX_TOKENS, 32 <= H <= MOE_MAX_DIM, H a multiple of 32. */
int moe_rmsnorm(const void *x, const void *gamma, int T, int H, float eps, void *y, int flags, void *stream);

/* Router scores and top-k in one launch (T <= 16; two launches beyond):
 *   logits[t][e] = sum_j router_w[e][j] * x[t][j]  (bf16 inputs, fp32 sums in
 *   a fixed order), then idx/w as moe_route_topk of those scores.
 * x: device bf16 [T][H]; router_w: device bf16 [E][H]; logits: device fp32
 * [T][E]; idx int32 / w fp32 [T][k].  ws: device, >= 256 bytes, zeroed once
 * (an arrival counter that the call returns to zero).  Limits as
 * moe_route_topk; H as moe_rmsnorm and at most 16384. */
int moe_router_topk_scores(const void *x, const void *router_w, int T, int H, int E, int k, float *logits,
                           int32_t *idx, float *w, void *ws, size_t ws_bytes, void *stream);

/* One MoE block: a layer plus the router and the norm in front of it. */
typedef struct moe_block {
    moe_layer layer;          /* the experts; hidden and n_experts also size the two arrays below */
    const void *norm_gamma;   /* device bf16 [hidden]: RMSNorm gains */
    const void *router_w;     /* device bf16 [n_experts][hidden]: router weights */
    float norm_eps;           /* RMSNorm epsilon, >= 0 */
    int32_t reserved;         /* must be 0 */
} moe_block;

/* Workspace of moe_block_decode for T tokens (0 when B or T breaks a rule):
 * the layer's workspace followed by the normalised activation and the scores. */
size_t moe_block_workspace_bytes(const moe_block *B, int T);

/* The whole block on the residual stream x (bf16 [T][hidden]):
 *   xn = bf16(RMSNorm(x)),  logits = router_w xn (fp32),
 *   out = x + moe_layer(xn, logits)  (the residual added before the layer's
 *   single rounding; bf16, or fp32 with MOE_OUT_F32).
 * Three launches (the norm, the scores, then the layer, which ranks the
 * scores itself: top-k fused with the experts); idx_out / w_out as
 * moe_layer_decode.  hidden <= 16384.  Other rules as moe_layer_decode. */
int moe_block_decode(const moe_block *B, const void *x, int T, void *out, int32_t *idx_out, float *w_out, int flags,
                     void *ws, size_t ws_bytes, void *stream);

/* Activation quantisation for the scaled matrix cores (the pages' fp6 path
 * with e4m3 activations: knivesysl README, "formats" and "key flags"; an amax
 * quantiser as Strata docs/INTEL.md, "The engine itself on Intel"): each
 * block of 32 consecutive elements of a row gets the UE8M0 scale 2^X with
 * X = floor(log2(max |x|)) - 8, clamped to [-127, 127] (-127 for a block of
 * zeros), and each element the e4m3 code nearest to x / 2^X (ties to even,
 * magnitudes past 448 saturated, sign kept).
 *   x: device bf16 [T][H], H a multiple of 32;  codes: device u8 [T][H];
 *   scales: device u8 [T][H/32]. */
int moe_quantize_mx_e4m3(const void *x, int T, int H, void *codes, void *scales, void *stream);

/* Dense block-scaled GEMV: y[b] = W x[b] for B tokens sharing every decoded
 * weight (knivesysl README, "formats": the fp6 projections).
 *   x: device bf16 [B][cols];  y: device [B][rows], bf16 or fp32 (MOE_OUT_F32)
 *   1 <= B <= MOE_MAX_GEMV_BATCH. */
int dense_gemv_q(const moe_qmat *W, const void *x, int B, void *y, int flags, void *stream);

/* Reads (synchronously, on `stream`) and clears the error word a kernel sets
 * in the workspace when a bounded inter-workgroup wait expires.  Returns
 * MOE_OK, MOE_EKERNEL, or a negative validation/HIP code. */
int moe_workspace_status(void *ws, size_t ws_bytes, void *stream);

/* Text of the last non-OK return on this thread ("" if none): the failing
 * argument and rule, or the HIP operation and its error (knivesysl README,
 * "current benchmark": native errors name the operation and the device error,
 * not only a number). */
const char *moe_last_error(void);

/* Library version, major * 10000 + minor * 100 + patch. */
int moe_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOEQ_H */
