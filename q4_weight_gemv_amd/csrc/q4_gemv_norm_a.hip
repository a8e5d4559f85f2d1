// Fused residual add + RMSNorm decode-product kernels for Q4_0, Q8_0 and Q1_0 (one token).
#include "q4_gemv_kernel.h"

namespace q4 {
namespace gemv {
template int dispatch_norm_cfg<FmtQ4_0>(const Cfg &, const uint8_t *, const float *, float *, int, int, hipStream_t,
                                        int, bool, const Prologue &);
template int dispatch_norm_cfg<FmtQ8_0>(const Cfg &, const uint8_t *, const float *, float *, int, int, hipStream_t,
                                        int, bool, const Prologue &);
template int dispatch_norm_cfg<FmtQ1_0>(const Cfg &, const uint8_t *, const float *, float *, int, int, hipStream_t,
                                        int, bool, const Prologue &);
}  // namespace gemv
}  // namespace q4
