// decode_e2m3_lut.hip -- the decode kernels for format e2m3, lut decoder.
#include "decode_inst.h"

MOEQ_DECODE_INSTANCE(FMT_E2M3, DEC_LUT)
