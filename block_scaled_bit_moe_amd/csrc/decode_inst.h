// decode_inst.h -- one (format, decoder) instantiation set of the three
// decode kernels (single token, 2..16 tokens, general), compiled in its own
// translation unit so the sets build in parallel.
#pragma once

#include "decode1_impl.h"
#include "decodeT_impl.h"
#include "decode_impl.h"

#define MOEQ_DECODE_INSTANCE(F, D)                                                                   \
    namespace moeq {                                                                                  \
    template <> DecodeFns decode_fns_for<F, D>() { return DecodeFns{decode_fd<F, D>, decode1_fd<F, D>, decodeT_fd<F, D>}; } \
    }
