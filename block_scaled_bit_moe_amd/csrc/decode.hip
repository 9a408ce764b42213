// decode.hip -- host side of the single-launch MoE decode: workspace size and
// dispatch to the (format, decoder) instantiations.
#include <stdlib.h>

#include "kernels.h"

namespace moeq {

template <> DecodeFns decode_fns_for<1, DEC_LUT>();
template <> DecodeFns decode_fns_for<1, DEC_HW>();
template <> DecodeFns decode_fns_for<2, DEC_LUT>();
template <> DecodeFns decode_fns_for<2, DEC_HW>();
template <> DecodeFns decode_fns_for<3, DEC_LUT>();
template <> DecodeFns decode_fns_for<3, DEC_HW>();
template <> DecodeFns decode_fns_for<4, DEC_LUT>();
template <> DecodeFns decode_fns_for<4, DEC_HW>();
template <> DecodeFns decode_fns_for<5, DEC_LUT>();
template <> DecodeFns decode_fns_for<5, DEC_HW>();

static DecodeFns fns_of(int fmt, int dec) {
    const bool hw = dec == DEC_HW;
    switch (fmt) {
        case 1: return hw ? decode_fns_for<1, DEC_HW>() : decode_fns_for<1, DEC_LUT>();
        case 2: return hw ? decode_fns_for<2, DEC_HW>() : decode_fns_for<2, DEC_LUT>();
        case 3: return hw ? decode_fns_for<3, DEC_HW>() : decode_fns_for<3, DEC_LUT>();
        case 4: return hw ? decode_fns_for<4, DEC_HW>() : decode_fns_for<4, DEC_LUT>();
        default: return hw ? decode_fns_for<5, DEC_HW>() : decode_fns_for<5, DEC_LUT>();
    }
}

// MOEQ_DECODE1=0 routes single-token calls, MOEQ_DECODET=0 routed calls of
// 2..16 tokens, to the general kernel (for A/B measurement; all give
// identical results).
static bool env_on(const char *name) {
    const char *v = getenv(name);
    return !(v && v[0] == '0');
}
static bool single_token_kernel_enabled() {
    static const bool on = env_on("MOEQ_DECODE1");
    return on;
}
static bool few_token_kernel_enabled() {
    static const bool on = env_on("MOEQ_DECODET");
    return on;
}

size_t decode_workspace_bytes(int T, int H, int I, int Ish, int k) {
    (void)T;
    (void)k;
    const size_t Imax = (size_t)(I > Ish ? I : Ish);
    // header | h words of the general kernel | its fp32 partials | tagged h words of the single-token kernel
    // | tagged h words and partial outputs of the few-token kernel
    return decode_quant_offset(H, I, Ish) + act_quant_bytes(DEC_MAX_T, H);
}

// The decode kernels' regions end here; the activation quantisation region
// (MOE_ACT_MXFP8) follows.
size_t decode_quant_offset(int H, int I, int Ish) {
    const size_t Imax = (size_t)(I > Ish ? I : Ish);
    const size_t end = WS_HEADER + (size_t)DEC_MAX_PAIRS * Imax * sizeof(uint32_t) + (size_t)DEC_MAX_PAIRS * H * sizeof(float) +
                       (size_t)33 * Imax * sizeof(uint64_t) + (size_t)DEC_MAX_PAIRS * (Imax + H) * sizeof(uint64_t);
    return (end + 255u) & ~(size_t)255u;
}

hipError_t launch_decode(const DecodeArgs &a0, int dec, hipStream_t s) {
    const DecodeFns f = fns_of(a0.L.fmt, dec);
    DecodeArgs a = a0;
    if (a0.act_mx) {
        // quantise the activations, then run the layer on their dequantised values
        uint8_t *q = a0.ws + decode_quant_offset(a0.L.H, a0.L.I, a0.L.Ish);
        const size_t n = (size_t)a0.T * a0.L.H;
        uint8_t *codes = q, *scales = q + ((n + 255u) & ~(size_t)255u);
        uint16_t *deq = reinterpret_cast<uint16_t *>(scales + ((n / 32 + 255u) & ~(size_t)255u));
        const hipError_t e = launch_mx_quant(a0.x, a0.T, a0.L.H, codes, scales, deq, s);
        if (e != hipSuccess) return e;
        a.x = deq;
    }
    if (a.T == 1 && a.mode == MODE_ROUTE && single_token_kernel_enabled()) {
        const hipError_t e = f.one(a, s);
        if (e != hipErrorNotSupported) return e;
        (void)hipGetLastError();
    }
    if (a.T >= 2 && a.T <= DEC_MAX_T && a.mode == MODE_ROUTE && few_token_kernel_enabled()) {
        const hipError_t e = f.few(a, s);
        if (e != hipErrorNotSupported) return e;
        (void)hipGetLastError();
    }
    return f.general(a, s);
}

}  // namespace moeq
