// gemv_e2m1.hip -- dense_gemv_q for format e2m1 (both decoders).
#include "gemv_impl.h"

MOEQ_GEMV_INSTANCE(FMT_E2M1)
