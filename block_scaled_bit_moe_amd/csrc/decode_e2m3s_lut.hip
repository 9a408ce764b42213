// decode_e2m3s_lut.hip -- the decode kernels for format e2m3s, lut decoder.
#include "decode_inst.h"

MOEQ_DECODE_INSTANCE(FMT_E2M3S, DEC_LUT)
