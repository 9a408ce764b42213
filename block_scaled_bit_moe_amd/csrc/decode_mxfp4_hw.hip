// decode_mxfp4_hw.hip -- the decode kernels for format mxfp4, hw decoder.
#include "decode_inst.h"

MOEQ_DECODE_INSTANCE(FMT_MXFP4, DEC_HW)
