// decode_e2m1_lut.hip -- the decode kernels for format e2m1, lut decoder.
#include "decode_inst.h"

MOEQ_DECODE_INSTANCE(FMT_E2M1, DEC_LUT)
