// abi.cpp -- the C ABI of include/moeq.h: argument validation (before anything
// is enqueued), dispatch to the kernels, thread-local error text.
// knivesysl README, introduction: the engine is one native library behind a C
// ABI that Python loads; its "current benchmark" section: native errors name
// the failing operation, not only a number.
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../include/moeq.h"
#include "kernels.h"

using namespace moeq;

static_assert(NOALLOC_SCRATCH_BYTES == MOE_NOALLOC_WORKSPACE_BYTES, "static workspace size");

static thread_local char g_err[512];

static int fail(int code, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

static int ok() {
    g_err[0] = 0;
    return MOE_OK;
}

static bool al16(const void *p) { return p && (((uintptr_t)p) & 15u) == 0; }

static bool fmt_known(int fmt) { return fmt >= MOE_FMT_E2M1_E4M3_B16 && fmt <= MOE_FMT_E2M3_E4M3_B16; }

// Dimensions must hold whole scale blocks and give 16-byte code rows.
static int block_of(int fmt) {
    switch (fmt) {
        case MOE_FMT_E2M1_E4M3_B16: return 32;
        case MOE_FMT_E2M3_UE8M0_B128: return 128;
        case MOE_FMT_E2M1_UE8M0_B32: return 32;
        case MOE_FMT_INT4_F16_B64: return 64;
        default: return 64;   // e2m3 + e4m3/16: 3*cols/4 bytes per row is a multiple of 16
    }
}

static int check_dim(const char *name, int v, int fmt) {
    const int b = block_of(fmt);
    if (v < b || v > MOE_MAX_DIM || v % b)
        return fail(MOE_EINVAL, "%s=%d must be a multiple of %d in [%d, %d] for format %d", name, v, b, b,
                    MOE_MAX_DIM, fmt);
    return MOE_OK;
}

static int check_ptr(const char *name, const void *p) {
    if (!p) return fail(MOE_EINVAL, "%s is NULL", name);
    if (!al16(p)) return fail(MOE_EINVAL, "%s=%p is not 16-byte aligned", name, p);
    return MOE_OK;
}

static int hip_fail(const char *op, hipError_t e) {
    return fail(MOE_EHIP, "%s: %s (%d)", op, hipGetErrorString(e), (int)e);
}

static int decoder_from_flags(int flags) {
    if (flags & MOE_DECODER_HW) return DEC_HW;
    if (flags & MOE_DECODER_LUT) return DEC_LUT;
    return decoder_choice();
}

int moeq::decoder_choice() {
    // read once (initialisation of a local static is thread-safe).  The
    // hardware conversions are the default: they decode a unit in fewer
    // instructions and leave LDS free; the table decoder stays selectable.
    static const int choice = [] {
        const char *v = getenv("MOEQ_DECODER");
        return (v && !strcmp(v, "lut")) ? DEC_LUT : DEC_HW;
    }();
    return choice;
}

#define CHECK(x)                         \
    do {                                 \
        int rc_ = (x);                   \
        if (rc_ != MOE_OK) return rc_;   \
    } while (0)

static int validate_layer(const moe_layer *L) {
    if (!L) return fail(MOE_EINVAL, "layer descriptor is NULL");
    if (!fmt_known(L->fmt)) return fail(MOE_EINVAL, "layer fmt=%d is not a known format", L->fmt);
    CHECK(check_dim("hidden", L->hidden, L->fmt));
    CHECK(check_dim("inter", L->inter, L->fmt));
    if (L->n_experts < 1 || L->n_experts > MOE_MAX_EXPERTS)
        return fail(MOE_EINVAL, "n_experts=%d must be in [1, %d]", L->n_experts, MOE_MAX_EXPERTS);
    const int kmax = L->n_experts < MOE_MAX_TOPK ? L->n_experts : MOE_MAX_TOPK;
    if (L->top_k < 1 || L->top_k > kmax)
        return fail(MOE_EINVAL, "top_k=%d must be in [1, min(n_experts, %d)=%d]", L->top_k, MOE_MAX_TOPK, kmax);
    if (L->shared_inter < 0) return fail(MOE_EINVAL, "shared_inter=%d is negative", L->shared_inter);
    CHECK(check_ptr("w13_codes", L->w13_codes));
    CHECK(check_ptr("w13_scales", L->w13_scales));
    CHECK(check_ptr("w2_codes", L->w2_codes));
    CHECK(check_ptr("w2_scales", L->w2_scales));
    if (L->shared_inter > 0) {
        CHECK(check_dim("shared_inter", L->shared_inter, L->fmt));
        CHECK(check_ptr("sh13_codes", L->sh13_codes));
        CHECK(check_ptr("sh13_scales", L->sh13_scales));
        CHECK(check_ptr("sh2_codes", L->sh2_codes));
        CHECK(check_ptr("sh2_scales", L->sh2_scales));
    }
    return MOE_OK;
}

static LayerArgs layer_args(const moe_layer *L) {
    LayerArgs a;
    a.w13c = (const uint8_t *)L->w13_codes;
    a.w13s = (const uint8_t *)L->w13_scales;
    a.w2c = (const uint8_t *)L->w2_codes;
    a.w2s = (const uint8_t *)L->w2_scales;
    a.sh13c = (const uint8_t *)L->sh13_codes;
    a.sh13s = (const uint8_t *)L->sh13_scales;
    a.sh2c = (const uint8_t *)L->sh2_codes;
    a.sh2s = (const uint8_t *)L->sh2_scales;
    a.fmt = L->fmt;
    a.H = L->hidden;
    a.I = L->inter;
    a.E = L->n_experts;
    a.k = L->top_k;
    a.Ish = L->shared_inter;
    return a;
}

static int decode_supported(const moe_layer *L, int T) {
    if (T > DEC_MAX_T) return MOE_OK;   // many-token path: no further limits
    if (L->hidden > DEC_MAX_DIM || L->inter > DEC_MAX_DIM || L->shared_inter > DEC_MAX_DIM)
        return fail(MOE_EUNSUPPORTED, "hidden/inter/shared_inter above %d are not supported by the decode kernels",
                    DEC_MAX_DIM);
    return MOE_OK;
}

static size_t ws_need(const moe_layer *L, int T) {
    if (T > DEC_MAX_T)
        return prefill_workspace_bytes(T, L->hidden, L->inter, L->shared_inter, L->top_k, L->n_experts);
    return decode_workspace_bytes(T, L->hidden, L->inter, L->shared_inter, L->top_k);
}

static hipError_t launch_layer(const DecodeArgs &a, int dec, hipStream_t s) {
    if (a.T > DEC_MAX_T) return launch_prefill(a, s);   // always the hardware decoder (same values)
    return launch_decode(a, dec, s);
}

extern "C" {

int moe_version(void) { return 100; }

const char *moe_last_error(void) { return g_err; }

int moe_route_topk(const float *logits, int T, int E, int k, int32_t *idx, float *w, void *stream) {
    CHECK(check_ptr("logits", logits));
    CHECK(check_ptr("idx", idx));
    CHECK(check_ptr("w", w));
    if (T < 1 || T > MOE_MAX_TOKENS) return fail(MOE_EINVAL, "T=%d must be in [1, %d]", T, MOE_MAX_TOKENS);
    if (E < 1 || E > MOE_MAX_EXPERTS) return fail(MOE_EINVAL, "E=%d must be in [1, %d]", E, MOE_MAX_EXPERTS);
    const int kmax = E < MOE_MAX_TOPK ? E : MOE_MAX_TOPK;
    if (k < 1 || k > kmax) return fail(MOE_EINVAL, "k=%d must be in [1, min(E, %d)=%d]", k, MOE_MAX_TOPK, kmax);
    hipError_t e = launch_route(logits, T, E, k, idx, w, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail("moe_route_topk launch", e);
    return ok();
}

size_t moe_layer_workspace_bytes(const moe_layer *L, int T) {
    if (validate_layer(L) != MOE_OK) return 0;
    if (T < 1 || T > MOE_MAX_TOKENS) {
        fail(MOE_EINVAL, "T=%d must be in [1, %d]", T, MOE_MAX_TOKENS);
        return 0;
    }
    if (decode_supported(L, T) != MOE_OK) return 0;
    ok();
    return ws_need(L, T);
}

static int check_ws(const moe_layer *L, int T, const void *ws, size_t ws_bytes) {
    if (!ws) return fail(MOE_EWORKSPACE, "workspace is NULL");
    if (((uintptr_t)ws) & 255u) return fail(MOE_EWORKSPACE, "workspace %p is not 256-byte aligned", ws);
    const size_t need = ws_need(L, T);
    if (ws_bytes < need) return fail(MOE_EWORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, need);
    return MOE_OK;
}

int moe_expert_ffn_q(const moe_layer *L, int expert, const void *x, int M, void *y, int flags, void *ws,
                     size_t ws_bytes, void *stream) {
    CHECK(validate_layer(L));
    if (expert < -1 || expert >= L->n_experts)
        return fail(MOE_EINVAL, "expert=%d must be -1 (shared) or in [0, %d)", expert, L->n_experts);
    if (expert == -1 && L->shared_inter <= 0) return fail(MOE_EINVAL, "expert=-1 but the layer has no shared expert");
    if (M < 1 || M > MOE_MAX_TOKENS) return fail(MOE_EINVAL, "M=%d must be in [1, %d]", M, MOE_MAX_TOKENS);
    CHECK(check_ptr("x", x));
    CHECK(check_ptr("y", y));
    CHECK(decode_supported(L, M));
    CHECK(check_ws(L, M, ws, ws_bytes));
    DecodeArgs a;
    memset(&a, 0, sizeof a);
    a.L = layer_args(L);
    a.x = (const uint16_t *)x;
    a.T = M;
    a.out = y;
    a.out_f32 = (flags & MOE_OUT_F32) ? 1 : 0;
    a.mode = expert < 0 ? MODE_FIXED_SHARED : MODE_FIXED_ROUTED;
    a.fixed_e = expert;
    a.ws = (uint8_t *)ws;
    a.spin_limit = (flags & MOE_DEBUG_SPIN_LIMIT) ? 0u : (1u << 20);
    a.act_mx = (flags & MOE_ACT_MXFP8) ? 1 : 0;
    hipError_t e = launch_layer(a, decoder_from_flags(flags), (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail("moe_expert_ffn_q launch", e);
    return ok();
}

int moe_layer_decode(const moe_layer *L, const void *x, const float *logits, int T, void *out, int32_t *idx_out,
                     float *w_out, int flags, void *ws, size_t ws_bytes, void *stream) {
    CHECK(validate_layer(L));
    if (T < 1 || T > MOE_MAX_TOKENS) return fail(MOE_EINVAL, "T=%d must be in [1, %d]", T, MOE_MAX_TOKENS);
    CHECK(check_ptr("x", x));
    CHECK(check_ptr("logits", logits));
    CHECK(check_ptr("out", out));
    if (idx_out && !al16(idx_out)) return fail(MOE_EINVAL, "idx_out is not 16-byte aligned");
    if (w_out && !al16(w_out)) return fail(MOE_EINVAL, "w_out is not 16-byte aligned");
    CHECK(decode_supported(L, T));
    CHECK(check_ws(L, T, ws, ws_bytes));
    DecodeArgs a;
    memset(&a, 0, sizeof a);
    a.L = layer_args(L);
    a.x = (const uint16_t *)x;
    a.logits = logits;
    a.T = T;
    a.out = out;
    a.idx_out = idx_out;
    a.w_out = w_out;
    a.out_f32 = (flags & MOE_OUT_F32) ? 1 : 0;
    a.mode = MODE_ROUTE;
    a.fixed_e = 0;
    a.ws = (uint8_t *)ws;
    a.spin_limit = (flags & MOE_DEBUG_SPIN_LIMIT) ? 0u : (1u << 20);
    a.act_mx = (flags & MOE_ACT_MXFP8) ? 1 : 0;
    hipError_t e = launch_layer(a, decoder_from_flags(flags), (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail("moe_layer_decode launch", e);
    return ok();
}

int moe_layer_decode_noalloc(const moe_layer *L, const void *x, const float *logits, int T, void *out,
                             int32_t *idx_out, float *w_out, int flags, void *stream) {
    CHECK(validate_layer(L));
    if (T < 1 || T > DEC_MAX_T)
        return fail(MOE_EINVAL, "T=%d must be in [1, %d] (the static workspace serves the decode path only)", T,
                    DEC_MAX_T);
    CHECK(check_ptr("x", x));
    CHECK(check_ptr("logits", logits));
    CHECK(check_ptr("out", out));
    if (idx_out && !al16(idx_out)) return fail(MOE_EINVAL, "idx_out is not 16-byte aligned");
    if (w_out && !al16(w_out)) return fail(MOE_EINVAL, "w_out is not 16-byte aligned");
    CHECK(decode_supported(L, T));
    const size_t need = ws_need(L, T);
    if (need > NOALLOC_SCRATCH_BYTES)
        return fail(MOE_EWORKSPACE, "this layer needs %zu bytes of workspace; the static workspace holds %zu", need,
                    (size_t)NOALLOC_SCRATCH_BYTES);
    void *ws = nullptr;
    const char *why = "";
    hipError_t e = noalloc_workspace((hipStream_t)stream, &ws, &why);
    if (e != hipSuccess) return fail(MOE_EHIP, "static workspace set-up: %s (%s)", why, hipGetErrorString(e));
    DecodeArgs a;
    memset(&a, 0, sizeof a);
    a.L = layer_args(L);
    a.x = (const uint16_t *)x;
    a.logits = logits;
    a.T = T;
    a.out = out;
    a.idx_out = idx_out;
    a.w_out = w_out;
    a.out_f32 = (flags & MOE_OUT_F32) ? 1 : 0;
    a.mode = MODE_ROUTE;
    a.fixed_e = 0;
    a.ws = (uint8_t *)ws;
    a.spin_limit = (flags & MOE_DEBUG_SPIN_LIMIT) ? 0u : (1u << 20);
    a.act_mx = (flags & MOE_ACT_MXFP8) ? 1 : 0;
    e = launch_decode(a, decoder_from_flags(flags), (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail("moe_layer_decode_noalloc launch", e);
    return ok();
}

static int check_rows(const char *name, int T, int H) {
    if (T < 1 || T > MOE_MAX_TOKENS) return fail(MOE_EINVAL, "%s: T=%d must be in [1, %d]", name, T, MOE_MAX_TOKENS);
    if (H < 32 || H > MOE_MAX_DIM || H % 32)
        return fail(MOE_EINVAL, "%s: H=%d must be a multiple of 32 in [32, %d]", name, H, MOE_MAX_DIM);
    return MOE_OK;
}

int moe_rmsnorm(const void *x, const void *gamma, int T, int H, float eps, void *y, int flags, void *stream) {
    CHECK(check_ptr("x", x));
    CHECK(check_ptr("gamma", gamma));
    CHECK(check_ptr("y", y));
    CHECK(check_rows("moe_rmsnorm", T, H));
    if (!(eps >= 0.f)) return fail(MOE_EINVAL, "eps=%g must be >= 0", (double)eps);
    hipError_t e = launch_rmsnorm((const uint16_t *)x, (const uint16_t *)gamma, T, H, eps, y,
                                  (flags & MOE_OUT_F32) ? 1 : 0, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail("moe_rmsnorm launch", e);
    return ok();
}

int moe_router_topk_scores(const void *x, const void *router_w, int T, int H, int E, int k, float *logits,
                           int32_t *idx, float *w, void *ws, size_t ws_bytes, void *stream) {
    CHECK(check_ptr("x", x));
    CHECK(check_ptr("router_w", router_w));
    CHECK(check_ptr("logits", logits));
    CHECK(check_ptr("idx", idx));
    CHECK(check_ptr("w", w));
    CHECK(check_rows("moe_router_topk_scores", T, H));
    if (H > ROUTER_MAX_H) return fail(MOE_EUNSUPPORTED, "H=%d above %d is not supported by the router kernel", H, ROUTER_MAX_H);
    if (E < 1 || E > MOE_MAX_EXPERTS) return fail(MOE_EINVAL, "E=%d must be in [1, %d]", E, MOE_MAX_EXPERTS);
    const int kmax = E < MOE_MAX_TOPK ? E : MOE_MAX_TOPK;
    if (k < 1 || k > kmax) return fail(MOE_EINVAL, "k=%d must be in [1, min(E, %d)=%d]", k, MOE_MAX_TOPK, kmax);
    if (!ws) return fail(MOE_EWORKSPACE, "workspace is NULL");
    if (((uintptr_t)ws) & 255u) return fail(MOE_EWORKSPACE, "workspace %p is not 256-byte aligned", ws);
    if (ws_bytes < 256) return fail(MOE_EWORKSPACE, "workspace has %zu bytes, needs 256", ws_bytes);
    hipError_t e = launch_router((const uint16_t *)x, (const uint16_t *)router_w, T, H, E, k, logits, idx, w,
                                 (uint32_t *)ws + WS_ROUTER_ARRIVE, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail("moe_router_topk_scores launch", e);
    return ok();
}

static size_t align256(size_t v) { return (v + 255u) & ~(size_t)255u; }

static int validate_block(const moe_block *B) {
    if (!B) return fail(MOE_EINVAL, "block descriptor is NULL");
    CHECK(validate_layer(&B->layer));
    CHECK(check_ptr("norm_gamma", B->norm_gamma));
    CHECK(check_ptr("router_w", B->router_w));
    if (!(B->norm_eps >= 0.f)) return fail(MOE_EINVAL, "norm_eps=%g must be >= 0", (double)B->norm_eps);
    if (B->reserved != 0) return fail(MOE_EINVAL, "block reserved field must be 0");
    return MOE_OK;
}

// block workspace: the layer's, then xn bf16 [T][H], then logits fp32 [T][E]
static size_t block_xn_offset(const moe_block *B, int T) { return align256(ws_need(&B->layer, T)); }
static size_t block_lg_offset(const moe_block *B, int T) {
    return block_xn_offset(B, T) + align256((size_t)T * B->layer.hidden * 2);
}
static size_t block_ws_need(const moe_block *B, int T) {
    return block_lg_offset(B, T) + align256((size_t)T * B->layer.n_experts * 4);
}

size_t moe_block_workspace_bytes(const moe_block *B, int T) {
    if (validate_block(B) != MOE_OK) return 0;
    if (T < 1 || T > MOE_MAX_TOKENS) {
        fail(MOE_EINVAL, "T=%d must be in [1, %d]", T, MOE_MAX_TOKENS);
        return 0;
    }
    if (decode_supported(&B->layer, T) != MOE_OK) return 0;
    ok();
    return block_ws_need(B, T);
}

int moe_block_decode(const moe_block *B, const void *x, int T, void *out, int32_t *idx_out, float *w_out, int flags,
                     void *ws, size_t ws_bytes, void *stream) {
    CHECK(validate_block(B));
    const moe_layer *L = &B->layer;
    if (T < 1 || T > MOE_MAX_TOKENS) return fail(MOE_EINVAL, "T=%d must be in [1, %d]", T, MOE_MAX_TOKENS);
    CHECK(check_ptr("x", x));
    CHECK(check_ptr("out", out));
    if (idx_out && !al16(idx_out)) return fail(MOE_EINVAL, "idx_out is not 16-byte aligned");
    if (w_out && !al16(w_out)) return fail(MOE_EINVAL, "w_out is not 16-byte aligned");
    CHECK(decode_supported(L, T));
    if (L->hidden > ROUTER_MAX_H)
        return fail(MOE_EUNSUPPORTED, "hidden=%d above %d is not supported by the router kernel", L->hidden, ROUTER_MAX_H);
    if (!ws) return fail(MOE_EWORKSPACE, "workspace is NULL");
    if (((uintptr_t)ws) & 255u) return fail(MOE_EWORKSPACE, "workspace %p is not 256-byte aligned", ws);
    const size_t need = block_ws_need(B, T);
    if (ws_bytes < need) return fail(MOE_EWORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, need);
    uint16_t *xn = (uint16_t *)((uint8_t *)ws + block_xn_offset(B, T));
    float *lg = (float *)((uint8_t *)ws + block_lg_offset(B, T));
    hipStream_t s = (hipStream_t)stream;
    // norm, then scores; the layer ranks them itself (top-k fused with the experts)
    hipError_t e = launch_rmsnorm((const uint16_t *)x, (const uint16_t *)B->norm_gamma, T, L->hidden, B->norm_eps, xn,
                                  0, s);
    if (e != hipSuccess) return hip_fail("moe_block_decode norm launch", e);
    e = launch_router(xn, (const uint16_t *)B->router_w, T, L->hidden, L->n_experts, L->top_k, lg, nullptr, nullptr,
                      nullptr, s);
    if (e != hipSuccess) return hip_fail("moe_block_decode scores launch", e);
    DecodeArgs a;
    memset(&a, 0, sizeof a);
    a.L = layer_args(L);
    a.x = xn;
    a.logits = lg;
    a.T = T;
    a.out = out;
    a.idx_out = idx_out;
    a.w_out = w_out;
    a.out_f32 = (flags & MOE_OUT_F32) ? 1 : 0;
    a.mode = MODE_ROUTE;
    a.ws = (uint8_t *)ws;
    a.spin_limit = (flags & MOE_DEBUG_SPIN_LIMIT) ? 0u : (1u << 20);
    a.act_mx = (flags & MOE_ACT_MXFP8) ? 1 : 0;
    a.residual = (const uint16_t *)x;
    e = launch_layer(a, decoder_from_flags(flags), s);
    if (e != hipSuccess) return hip_fail("moe_block_decode layer launch", e);
    return ok();
}

int moe_quantize_mx_e4m3(const void *x, int T, int H, void *codes, void *scales, void *stream) {
    CHECK(check_ptr("x", x));
    CHECK(check_ptr("codes", codes));
    CHECK(check_ptr("scales", scales));
    CHECK(check_rows("moe_quantize_mx_e4m3", T, H));
    hipError_t e = launch_mx_quant((const uint16_t *)x, T, H, (uint8_t *)codes, (uint8_t *)scales, nullptr,
                                   (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail("moe_quantize_mx_e4m3 launch", e);
    return ok();
}

int dense_gemv_q(const moe_qmat *W, const void *x, int B, void *y, int flags, void *stream) {
    if (!W) return fail(MOE_EINVAL, "matrix descriptor is NULL");
    if (!fmt_known(W->fmt)) return fail(MOE_EINVAL, "matrix fmt=%d is not a known format", W->fmt);
    if (W->reserved != 0) return fail(MOE_EINVAL, "matrix reserved field must be 0");
    if (W->rows < 1 || W->rows > (1 << 24)) return fail(MOE_EINVAL, "rows=%d must be in [1, %d]", W->rows, 1 << 24);
    CHECK(check_dim("cols", W->cols, W->fmt));
    if (W->cols > DEC_MAX_DIM)
        return fail(MOE_EUNSUPPORTED, "cols=%d above %d is not supported by the GEMV kernel", W->cols, DEC_MAX_DIM);
    if (B < 1 || B > MOE_MAX_GEMV_BATCH) return fail(MOE_EINVAL, "B=%d must be in [1, %d]", B, MOE_MAX_GEMV_BATCH);
    CHECK(check_ptr("codes", W->codes));
    CHECK(check_ptr("scales", W->scales));
    CHECK(check_ptr("x", x));
    CHECK(check_ptr("y", y));
    hipError_t e = launch_gemv(W->fmt, decoder_from_flags(flags), (const uint8_t *)W->codes,
                               (const uint8_t *)W->scales, W->rows, W->cols, (const uint16_t *)x, B, y,
                               (flags & MOE_OUT_F32) ? 1 : 0, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail("dense_gemv_q launch", e);
    return ok();
}

int moe_workspace_status(void *ws, size_t ws_bytes, void *stream) {
    if (!ws) return fail(MOE_EWORKSPACE, "workspace is NULL");
    if (ws_bytes < WS_HEADER) return fail(MOE_EWORKSPACE, "workspace has %zu bytes, needs at least %zu", ws_bytes,
                                          (size_t)WS_HEADER);
    uint32_t err = 0;
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = hipMemcpyAsync(&err, ws, sizeof err, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail("moe_workspace_status read", e);
    if (err) {
        e = hipMemsetAsync(ws, 0, sizeof err, s);
        if (e == hipSuccess) e = hipStreamSynchronize(s);
        if (e != hipSuccess) return hip_fail("moe_workspace_status clear", e);
        return fail(MOE_EKERNEL, "a kernel's bounded inter-workgroup wait expired; its output is invalid");
    }
    return ok();
}

}  // extern "C"
