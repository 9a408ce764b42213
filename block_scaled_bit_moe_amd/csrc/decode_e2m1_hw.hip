// decode_e2m1_hw.hip -- one (format, decoder) instantiation set of the
// single-launch MoE decode kernel (decode_impl.h), compiled on its own.
#include "decode1_impl.h"
#include "decodeT_impl.h"
#include "decode_impl.h"

namespace moeq {
hipError_t decode_launch_e2m1_hw(const DecodeArgs &a, hipStream_t s) { return decode_fd<FMT_E2M1, DEC_HW>(a, s); }
hipError_t decode1_launch_e2m1_hw(const DecodeArgs &a, hipStream_t s) { return decode1_fd<FMT_E2M1, DEC_HW>(a, s); }
hipError_t decodeT_launch_e2m1_hw(const DecodeArgs &a, hipStream_t s) { return decodeT_fd<FMT_E2M1, DEC_HW>(a, s); }
}  // namespace moeq
