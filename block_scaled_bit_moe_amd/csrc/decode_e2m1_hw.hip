// decode_e2m1_hw.hip -- the decode kernels for format e2m1, hw decoder.
#include "decode_inst.h"

MOEQ_DECODE_INSTANCE(FMT_E2M1, DEC_HW)
