// Internal declarations shared by the host launchers of the library.
#pragma once

#include <cstddef>
#include <cstdint>

#include "q4.h"

namespace q4 {

// Units: every kernel works on "units" of 32 weights = 16 nibble bytes.
// Q4_0: one block. Q4_K: one eighth of a 256-weight super-block.
constexpr int kUnitWeights = 32;

// Validation shared by the device entry points. Returns Q4_OK or the status
// to report; makes no HIP call.
int check_product_args(int fmt, const void *w, const void *x, const float *y,
                       int64_t m, int64_t k, int64_t n, int64_t n_max);

// Launch one decode product (arguments already validated).
int launch_gemv(int fmt, const void *w, const float *x, float *y,
                int64_t m, int64_t k, int64_t n, void *stream);

// Launch one prefill product (arguments already validated).
int launch_gemm(int fmt, const void *w, const uint16_t *x, float *y,
                int64_t m, int64_t k, int64_t n, void *stream);

}  // namespace q4
