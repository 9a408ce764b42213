// gemv_mxfp4.hip -- dense_gemv_q for format mxfp4 (both decoders).
#include "gemv_impl.h"

MOEQ_GEMV_INSTANCE(FMT_MXFP4)
