// Fused residual add + RMSNorm decode-product kernels for Q4_K and Q2_K (one token).
#include "q4_gemv_kernel.h"

namespace q4 {
namespace gemv {
template int dispatch_norm_cfg<FmtQ4_K>(const Cfg &, const uint8_t *, const float *, float *, int, int, hipStream_t,
                                        int, bool, const Prologue &);
template int dispatch_norm_cfg<FmtQ2_K>(const Cfg &, const uint8_t *, const float *, float *, int, int, hipStream_t,
                                        int, bool, const Prologue &);
}  // namespace gemv
}  // namespace q4
