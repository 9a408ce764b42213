// decode.hip -- host side of the single-launch MoE decode: workspace size and
// dispatch to the (format, decoder) instantiations.
#include "kernels.h"

namespace moeq {

hipError_t decode_launch_e2m1_lut(const DecodeArgs &a, hipStream_t s);
hipError_t decode_launch_e2m1_hw(const DecodeArgs &a, hipStream_t s);
hipError_t decode_launch_e2m3_lut(const DecodeArgs &a, hipStream_t s);
hipError_t decode_launch_e2m3_hw(const DecodeArgs &a, hipStream_t s);

size_t decode_workspace_bytes(int T, int H, int I, int Ish, int k) {
    (void)T;
    (void)k;
    const size_t Imax = (size_t)(I > Ish ? I : Ish);
    return WS_HEADER + (size_t)DEC_MAX_PAIRS * Imax * sizeof(uint32_t) + (size_t)DEC_MAX_PAIRS * H * sizeof(float);
}

hipError_t launch_decode(const DecodeArgs &a, int dec, hipStream_t s) {
    if (a.L.fmt == 1) return dec == DEC_HW ? decode_launch_e2m1_hw(a, s) : decode_launch_e2m1_lut(a, s);
    return dec == DEC_HW ? decode_launch_e2m3_hw(a, s) : decode_launch_e2m3_lut(a, s);
}

}  // namespace moeq
