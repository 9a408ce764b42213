// decode_mxfp4_lut.hip -- the decode kernels for format mxfp4, lut decoder.
#include "decode_inst.h"

MOEQ_DECODE_INSTANCE(FMT_MXFP4, DEC_LUT)
