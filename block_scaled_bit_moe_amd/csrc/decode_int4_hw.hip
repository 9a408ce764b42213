// decode_int4_hw.hip -- the decode kernels for format int4, hw decoder.
#include "decode_inst.h"

MOEQ_DECODE_INSTANCE(FMT_INT4, DEC_HW)
