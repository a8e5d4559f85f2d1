// Prefill product Y = bf16(W_hat) X for 4-bit block-quantized W on gfx950.
#include <hip/hip_runtime.h>

#include "q4_internal.h"

namespace q4 {

int launch_gemm(int, const void *, const uint16_t *, float *, int64_t, int64_t, int64_t, void *)
{
    return Q4_EUNSUPPORTED;
}

}  // namespace q4

extern "C" int q4_gemm(int fmt, const void *w, const uint16_t *x_bf16, float *y, int64_t m, int64_t k, int64_t n,
                       void *hip_stream)
{
    int st = q4::check_product_args(fmt, w, x_bf16, y, m, k, n, INT64_MAX);
    if (st != Q4_OK) return st;
    if (m == 0 || n == 0) return Q4_OK;
    return q4::launch_gemm(fmt, w, x_bf16, y, m, k, n, hip_stream);
}
