// gemv_e2m3.hip -- dense_gemv_q for format e2m3 (both decoders).
#include "gemv_impl.h"

MOEQ_GEMV_INSTANCE(FMT_E2M3)
