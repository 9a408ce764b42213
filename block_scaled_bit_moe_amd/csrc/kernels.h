// kernels.h -- launchers of the gfx950 kernels (host side of each .hip file).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moeq {

// Decoder choice: LUT = tables in LDS indexed by whole bytes / 12-bit code
// pairs; HW = gfx950's scaled fp4/fp6 -> bf16 conversion instructions.  Both
// are exact; which is faster is measured.
constexpr int DEC_LUT = 0;
constexpr int DEC_HW = 1;

struct LayerArgs {
    const uint8_t *w13c, *w13s, *w2c, *w2s;       // routed experts, stacked
    const uint8_t *sh13c, *sh13s, *sh2c, *sh2s;   // shared expert (Ish > 0)
    int fmt, H, I, E, k, Ish;
};

enum { MODE_ROUTE = 0, MODE_FIXED_ROUTED = 1, MODE_FIXED_SHARED = 2 };

struct DecodeArgs {
    LayerArgs L;
    const uint16_t *x;        // bf16 [T][H]
    const float *logits;      // fp32 [T][E]  (MODE_ROUTE)
    int T;
    void *out;                // [T][H] bf16 or fp32
    int32_t *idx_out;         // nullable
    float *w_out;             // nullable
    int out_f32;
    int mode, fixed_e;
    uint8_t *ws;
    uint32_t spin_limit;
    const uint16_t *residual;   // bf16 [T][H] added to the output before its rounding (nullable)
    int act_mx;                 // quantise the activations to MX e4m3 (per 32) before gate | up
};

// Activation quantisation (quant.hip): bf16 [T][H] -> MX e4m3 codes [T][H]
// and UE8M0 scales [T][H/32]; deq (nullable) receives the dequantised bf16.
hipError_t launch_mx_quant(const uint16_t *x, int T, int H, uint8_t *codes, uint8_t *scales, uint16_t *deq,
                           hipStream_t s);
// Workspace bytes of that region for T tokens: codes, scales, dequantised rows.
inline size_t act_quant_bytes(int T, int H) {
    auto al = [](size_t v) { return (v + 255u) & ~(size_t)255u; };
    return al((size_t)T * H) + al((size_t)T * H / 32) + al((size_t)T * H * 2);
}

// decode-path workspace: header (counters, error word) + h (hi/lo bf16) + y partials
constexpr size_t WS_HEADER = 16384;
constexpr int WS_ERR = 0;          // u32 offsets into the header
constexpr int WS_EXIT = 1;
constexpr int WS_ARRIVE = 2;
constexpr int WS_EPOCH = 3;       // single-token kernel: calls completed on this workspace
constexpr int WS_GU = 16;          // gu_done[<= 1024]
constexpr int WS_DN = 16 + 1024;   // dn_done[<= 3072]
constexpr int DEC_MAX_T = 16;
constexpr int DEC_MAX_GROUPS = DEC_MAX_T * 32 + 1;
constexpr int DEC_MAX_PAIRS = DEC_MAX_T * 33;
constexpr int DEC_MAX_DIM = 8192;  // H, I, Ish on the decode path (x/h held in registers)
constexpr int DEC_S1 = 16;         // I-rows (gate and up) per gate/up item
constexpr int DEC_S2 = 64;         // output rows per down item

size_t decode_workspace_bytes(int T, int H, int I, int Ish, int k);
size_t decode_quant_offset(int H, int I, int Ish);

// Many-token path (T > DEC_MAX_T): tokens are processed in chunks of PF_CHUNK.
constexpr int PF_CHUNK = 2048;
size_t prefill_workspace_bytes(int T, int H, int I, int Ish, int k, int E);
hipError_t launch_prefill(const DecodeArgs &a, hipStream_t s);

// Lanes per row of the down projection: one mapping for every expert of the
// layer (set by the smaller intermediate size), so a token's arithmetic does
// not depend on which kernel or which other tokens share the call.
__host__ __device__ inline int down_lanes_per_row(int I, int Ish) {
    const int m = (Ish > 0 && Ish < I) ? Ish : I;
    int U = m / 32, l = 64;
    while (l > U && l > 1) l >>= 1;
    return l;
}

hipError_t launch_route(const float *logits, int T, int E, int k, int32_t *idx, float *w, hipStream_t s);

// The steps either side of the layer (block.hip).  launch_rmsnorm: y = x g /
// sqrt(mean x^2 + eps) per row.  launch_router: scores of router weights wr
// [E][H] (bf16) for T tokens, then with idx/w the top-k (in the same launch
// for T <= 16, using the arrival counter, which must be zero between calls).
constexpr int WS_ROUTER_ARRIVE = 5;   // header word of that counter
constexpr int ROUTER_MAX_H = 16384;   // hidden sizes the router kernel takes
hipError_t launch_rmsnorm(const uint16_t *x, const uint16_t *g, int T, int H, float eps, void *y, int out_f32,
                          hipStream_t s);
hipError_t launch_router(const uint16_t *x, const uint16_t *wr, int T, int H, int E, int k, float *logits,
                         int32_t *idx, float *w, uint32_t *counter, hipStream_t s);
hipError_t launch_gemv(int fmt, int dec, const uint8_t *codes, const uint8_t *scales, int rows, int cols,
                       const uint16_t *x, int B, void *y, int out_f32, hipStream_t s);
hipError_t launch_decode(const DecodeArgs &a, int dec, hipStream_t s);

// The dense GEMV of one (format, decoder) pair (gemv_<format>.hip).
typedef hipError_t (*GemvFn)(const uint8_t *codes, const uint8_t *scales, int rows, int cols, const uint16_t *x,
                             int B, void *y, int out_f32, hipStream_t s);
template <int FMT, int DEC> GemvFn gemv_fn_for();

// The decode launchers of one (format, decoder) pair, each defined in its own
// translation unit (decode_<format>_<decoder>.hip).  A launcher returns
// hipErrorNotSupported when the call's shape is outside what its kernel takes.
typedef hipError_t (*DecodeFn)(const DecodeArgs &, hipStream_t);
struct DecodeFns {
    DecodeFn general;   // any T <= 16, fixed-expert calls
    DecodeFn one;       // T == 1
    DecodeFn few;       // 2 <= T <= 16
};
template <int FMT, int DEC> DecodeFns decode_fns_for();

int decoder_choice();    // DEC_LUT or DEC_HW (MOEQ_DECODER=lut|hw, read once)

// The library-owned workspace of moe_layer_decode_noalloc (noalloc.hip): a
// static device array per GPU.  noalloc_workspace gives its address on the
// current device (cleared on the first call there, which must not be under
// graph capture).
constexpr size_t NOALLOC_SCRATCH_BYTES = (size_t)64 << 20;
constexpr int NOALLOC_MAX_DEVICES = 64;
hipError_t noalloc_workspace(hipStream_t s, void **ptr, const char **why);

// Cached runtime queries (launch_cache.cpp), per device; thread-safe.
int current_device();
int cached_cus();                                                  // CUs of the current device
int cached_occupancy(const void *kern, int threads, size_t dyn);   // resident workgroups per CU
hipError_t ensure_dyn_lds(const void *kern, size_t dyn);           // allow `dyn` bytes of dynamic LDS

}  // namespace moeq
