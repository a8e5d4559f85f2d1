// The one-token streaming decode kernel (q4_gemv_stream.h), instantiated for
// every format over its geometries (lanes per row, waves per workgroup, weight
// slots in flight per lane), plain and with the fused add + RMSNorm prologue.
#include "q4_gemv_stream.h"

namespace q4 {
namespace gemv {

// The instantiated streaming geometries: (lanes per row, waves per group, depth).
#define Q4_STREAM_CONFIGS(X) \
    X(8, 16, 2)              \
    X(16, 16, 2)             \
    X(16, 1, 2)              \
    X(32, 1, 2)              \
    X(32, 8, 2)              \
    X(32, 16, 2)             \
    X(64, 4, 2)              \
    X(64, 8, 2)              \
    X(64, 16, 2)             \
    X(64, 8, 3)              \
    X(64, 16, 4)

template <class F>
int dispatch_stream(const Cfg &c, const uint8_t *w, const float *x, float *y, int m, int k, hipStream_t s, int cus)
{
    if (c.r != 1 && c.r != 0) return Q4_EUNSUPPORTED;
#define Q4_STREAM_CASE(L, WV, DD) \
    if (c.lpr == L && c.waves == WV && c.depth == DD) return launch_stream<F, L, WV, DD>(w, x, y, m, k, s, cus, c.groups_per_cu);
    Q4_STREAM_CONFIGS(Q4_STREAM_CASE)
#undef Q4_STREAM_CASE
    return Q4_EUNSUPPORTED;
}

template <class F>
int dispatch_stream_norm(const Cfg &c, const uint8_t *w, const float *x, float *y, int m, int k, hipStream_t s,
                         int cus, const Prologue &pro)
{
    if (c.r != 1 && c.r != 0) return Q4_EUNSUPPORTED;
#define Q4_STREAM_CASE(L, WV, DD)                                                                   \
    if (c.lpr == L && c.waves == WV && c.depth == DD)                                               \
        return launch_stream<F, L, WV, DD, true>(w, x, y, m, k, s, cus, c.groups_per_cu, pro);
    Q4_STREAM_CONFIGS(Q4_STREAM_CASE)
#undef Q4_STREAM_CASE
    return Q4_EUNSUPPORTED;
}

template int dispatch_stream<FmtQ4_0>(const Cfg &, const uint8_t *, const float *, float *, int, int, hipStream_t, int);
template int dispatch_stream<FmtQ8_0>(const Cfg &, const uint8_t *, const float *, float *, int, int, hipStream_t, int);
template int dispatch_stream<FmtQ1_0>(const Cfg &, const uint8_t *, const float *, float *, int, int, hipStream_t, int);
template int dispatch_stream<FmtQ4_K>(const Cfg &, const uint8_t *, const float *, float *, int, int, hipStream_t, int);
template int dispatch_stream<FmtQ2_K>(const Cfg &, const uint8_t *, const float *, float *, int, int, hipStream_t, int);

template int dispatch_stream_norm<FmtQ4_0>(const Cfg &, const uint8_t *, const float *, float *, int, int, hipStream_t, int,
                                         const Prologue &);
template int dispatch_stream_norm<FmtQ8_0>(const Cfg &, const uint8_t *, const float *, float *, int, int, hipStream_t, int,
                                         const Prologue &);
template int dispatch_stream_norm<FmtQ1_0>(const Cfg &, const uint8_t *, const float *, float *, int, int, hipStream_t, int,
                                         const Prologue &);
template int dispatch_stream_norm<FmtQ4_K>(const Cfg &, const uint8_t *, const float *, float *, int, int, hipStream_t, int,
                                         const Prologue &);
template int dispatch_stream_norm<FmtQ2_K>(const Cfg &, const uint8_t *, const float *, float *, int, int, hipStream_t, int,
                                         const Prologue &);

}  // namespace gemv
}  // namespace q4
