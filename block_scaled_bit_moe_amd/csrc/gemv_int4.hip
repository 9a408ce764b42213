// gemv_int4.hip -- dense_gemv_q for format int4 (both decoders).
#include "gemv_impl.h"

MOEQ_GEMV_INSTANCE(FMT_INT4)
