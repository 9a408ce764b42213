// decode_e2m3s_hw.hip -- the decode kernels for format e2m3s, hw decoder.
#include "decode_inst.h"

MOEQ_DECODE_INSTANCE(FMT_E2M3S, DEC_HW)
