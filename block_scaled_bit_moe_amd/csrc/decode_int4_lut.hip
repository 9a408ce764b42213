// decode_int4_lut.hip -- the decode kernels for format int4, lut decoder.
#include "decode_inst.h"

MOEQ_DECODE_INSTANCE(FMT_INT4, DEC_LUT)
