// gemv_e2m3s.hip -- dense_gemv_q for format e2m3s (both decoders).
#include "gemv_impl.h"

MOEQ_GEMV_INSTANCE(FMT_E2M3S)
