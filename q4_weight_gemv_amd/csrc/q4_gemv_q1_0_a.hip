// Decode-product kernels for Q1_0, token counts 1..4 (split across units so they compile in parallel).
#include "q4_gemv_kernel.h"

namespace q4 {
namespace gemv {
template int dispatch_cfg<FmtQ1_0, 1>(const Cfg &, const uint8_t *, const float *, float *, int, int, hipStream_t, int);
template int dispatch_cfg<FmtQ1_0, 2>(const Cfg &, const uint8_t *, const float *, float *, int, int, hipStream_t, int);
template int dispatch_cfg<FmtQ1_0, 3>(const Cfg &, const uint8_t *, const float *, float *, int, int, hipStream_t, int);
template int dispatch_cfg<FmtQ1_0, 4>(const Cfg &, const uint8_t *, const float *, float *, int, int, hipStream_t, int);
template int dispatch_glu_cfg<FmtQ1_0, 1>(const Cfg &, const uint8_t *, const float *, float *, int, int, hipStream_t, int);
template int dispatch_glu_cfg<FmtQ1_0, 2>(const Cfg &, const uint8_t *, const float *, float *, int, int, hipStream_t, int);
template int dispatch_glu_cfg<FmtQ1_0, 3>(const Cfg &, const uint8_t *, const float *, float *, int, int, hipStream_t, int);
template int dispatch_glu_cfg<FmtQ1_0, 4>(const Cfg &, const uint8_t *, const float *, float *, int, int, hipStream_t, int);
}  // namespace gemv
}  // namespace q4
