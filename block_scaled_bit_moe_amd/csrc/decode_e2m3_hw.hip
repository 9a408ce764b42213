// decode_e2m3_hw.hip -- the decode kernels for format e2m3, hw decoder.
#include "decode_inst.h"

MOEQ_DECODE_INSTANCE(FMT_E2M3, DEC_HW)
