// gemv.hip -- dense_gemv_q dispatch to the per-format instantiations
// (gemv_<format>.hip, each compiled on its own).
#include "kernels.h"

namespace moeq {

template <> GemvFn gemv_fn_for<1, DEC_HW>();
template <> GemvFn gemv_fn_for<1, DEC_LUT>();
template <> GemvFn gemv_fn_for<2, DEC_HW>();
template <> GemvFn gemv_fn_for<2, DEC_LUT>();
template <> GemvFn gemv_fn_for<3, DEC_HW>();
template <> GemvFn gemv_fn_for<3, DEC_LUT>();
template <> GemvFn gemv_fn_for<4, DEC_HW>();
template <> GemvFn gemv_fn_for<4, DEC_LUT>();
template <> GemvFn gemv_fn_for<5, DEC_HW>();
template <> GemvFn gemv_fn_for<5, DEC_LUT>();

hipError_t launch_gemv(int fmt, int dec, const uint8_t *codes, const uint8_t *scales, int rows, int cols,
                       const uint16_t *x, int B, void *y, int out_f32, hipStream_t s) {
    const bool hw = dec == DEC_HW;
    GemvFn f;
    switch (fmt) {
        case 1: f = hw ? gemv_fn_for<1, DEC_HW>() : gemv_fn_for<1, DEC_LUT>(); break;
        case 2: f = hw ? gemv_fn_for<2, DEC_HW>() : gemv_fn_for<2, DEC_LUT>(); break;
        case 3: f = hw ? gemv_fn_for<3, DEC_HW>() : gemv_fn_for<3, DEC_LUT>(); break;
        case 4: f = hw ? gemv_fn_for<4, DEC_HW>() : gemv_fn_for<4, DEC_LUT>(); break;
        default: f = hw ? gemv_fn_for<5, DEC_HW>() : gemv_fn_for<5, DEC_LUT>(); break;
    }
    return f(codes, scales, rows, cols, x, B, y, out_f32, s);
}

}  // namespace moeq
