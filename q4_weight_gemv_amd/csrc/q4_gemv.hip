// Host side of the decode product: argument checks, tile-geometry choice and
// the q4_gemv / q4_gemv_tuned entry points. The kernels themselves live in
// q4_gemv_kernel.h, instantiated per format in q4_gemv_q4_*.hip.
//
// Tile and workgroup sizes are tunable parameters with defaults picked by a
// sweep on the target device (Llamas on the Web, technical summary,
// Methodology section 2, "tunable parameters"); here the target is one chip,
// gfx950, so the defaults below encode the sweep's outcome for it.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>

#include "q4_internal.h"

namespace q4 {

namespace {
thread_local hipError_t last_hip_error = hipSuccess;
}

int hip_status(hipError_t e)
{
    if (e == hipSuccess) return Q4_OK;
    last_hip_error = e;
    return Q4_EHIP;
}

int device_cus()
{
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hip_status(hipGetDevice(&dev)) != Q4_OK) return -1;
    if (dev >= 0 && dev < 64) {
        int v = cache[dev].load(std::memory_order_relaxed);
        if (v > 0) return v;
    }
    int cus = 0;
    if (hip_status(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != Q4_OK || cus <= 0)
        return -1;
    if (dev >= 0 && dev < 64) cache[dev].store(cus, std::memory_order_relaxed);
    return cus;
}

int device_lds_optin()
{
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hip_status(hipGetDevice(&dev)) != Q4_OK) return -1;
    if (dev >= 0 && dev < 64) {
        const int v = cache[dev].load(std::memory_order_relaxed);
        if (v != 0) return v;
    }
    int bytes = 0;
    if (hipDeviceGetAttribute(&bytes, hipDeviceAttributeSharedMemPerBlockOptin, dev) != hipSuccess || bytes <= 0)
        bytes = -1;
    if (dev >= 0 && dev < 64) cache[dev].store(bytes, std::memory_order_relaxed);
    return bytes;
}

namespace gemv {

// Default geometries, from sweeps of every instantiated geometry on gfx950
// (cold weights, graph-replayed launches) at the decode shapes of the
// GPT-2-124M and SmolLM2-360M steps and the 7B-class layer, per format and
// token count. The tiled kernel (several tokens, the gated and fused-norm
// products, and one token where the streaming kernel is not chosen), rows
// of nu 32-weight units:
//   Q4_0, one token: nu <= 32 -> one-wave groups, 32 lanes per row, two rows
//     per lane (LM heads, m >= 16384: 8 lanes x 1 row); nu < 128 -> 4 waves,
//     64 lanes per row; longer rows -> 4 waves, 32 lanes x 2 rows.
//   Q4_0, several tokens: 4 waves; 64 lanes per row for 33..127 units, else
//     32 lanes x 2 rows; at 6..8 tokens of 128..255 units, 8-wave groups of
//     one row per lane (the whole row's activations in the opt-in LDS); the
//     same for Q8_0 and Q1_0.
//   Q2_K: the Q4_K choices for rows of fewer than 128 units; longer rows:
//     32 lanes x 2 rows in 4-wave groups (8-wave groups of one row per lane
//     at one token for rows of 256 units or more, and at 6..8 tokens for rows
//     of 128..255 units).
//   Q1_0: the Q4_0 choices, except two rows per lane for one-token LM
//     heads (m >= 16384, nu <= 32: 8 lanes x 2 rows).
//   Q8_0: the Q4_0 choices (same unit of 32 weights, twice the bytes),
//     except one row per lane at one token for rows of 128 units or more
//     (4 waves; 64 lanes per row for tall products, else 32).
//   Q4_K: 4 waves of 64 lanes per row for 33..127 units. Short rows: 16
//     lanes per row, one-wave groups at 1..2 tokens, 4 waves at 3..4, and 32
//     lanes x 2 rows from 5 tokens. Rows of 256 units or more, and rows of
//     128..255 units at several tokens: 8-wave groups of 32 lanes per row.
//     Rows of 128..255 units at one token: the same 8-wave groups for tall
//     products, else 4 waves of 16 lanes per row.
//   One token, rows of up to kStreamMaxUnits units, every format: the
//     streaming kernel (two weight slots in flight per lane), from a sweep of
//     its geometries and the tiled choice at the workload shapes
//     (bench.py --sweep; 256 compute units): short rows (nu <= 32) 32 lanes
//     per row in one 8-wave group per compute unit, LM heads (m >= 16384)
//     8 (nu <= 24, and Q1_0) or 16 lanes per row in 16-wave groups (Q8_0:
//     32); longer rows 64 lanes per row: one 8-wave group per compute unit
//     below 8 rows per compute unit, two from 8 to 16 rows per compute unit
//     of rows up to 4096 weights (and for every longer Q8_0 row), else one
//     16-wave group. Q8_0's short rows below LM-head height stay on the
//     tiled kernel (within 2 % either way).
Cfg choose_stream(int fmt, int64_t m, int64_t k, int cus)
{
    const int64_t nu = k / kUnitWeights;
    if (nu <= 32) {
        if (m >= 16384) {
            if (fmt == Q4_FMT_Q8_0) return Cfg{32, 1, 16, 1, 2};
            return Cfg{nu <= 24 || fmt == Q4_FMT_Q1_0 ? 8 : 16, 1, 16, 1, 2};
        }
        return Cfg{32, 1, 8, 1, 2};
    }
    if (m < 8LL * cus) return Cfg{64, 1, 8, 1, 2};
    if ((nu <= 128 && m <= 16LL * cus) || fmt == Q4_FMT_Q8_0) return Cfg{64, 1, 8, 2, 2};
    return Cfg{64, 1, 16, 1, 2};
}

Cfg choose_tiled(int fmt, int64_t m, int64_t k, int64_t n, int cus);

// The Q4_K matrix-core kernel from several tokens on, for products of 256
// rows or more (one fp16 per activation, as the tiled kernel there). From a
// sweep against the tiled kernel's per-token dot products: faster from 3
// tokens on at every measured shape, plain and gated; at 2 tokens only on
// rows of up to 2048 weights.
bool use_matrix(int fmt, int64_t m, int64_t k, int64_t n)
{
    return fmt == Q4_FMT_Q4_K && m >= 256 && (n >= 3 || (n == 2 && k <= 2048));
}

Cfg choose(int fmt, int64_t m, int64_t k, int64_t n, int cus)
{
    if (use_matrix(fmt, m, k, n)) {
        Cfg c{0, 0, 0, 1};
        c.matrix = true;
        return c;
    }
    const int64_t nu = k / kUnitWeights;
    const bool q8_short = fmt == Q4_FMT_Q8_0 && nu <= 32 && m < 16384;
    if (n == 1 && nu <= kStreamMaxUnits && !q8_short) return choose_stream(fmt, m, k, cus);
    return choose_tiled(fmt, m, k, n, cus);
}

Cfg choose_tiled(int fmt, int64_t m, int64_t k, int64_t n, int cus)
{
    (void)cus;
    const int64_t nu = k / kUnitWeights;
    if (fmt == Q4_FMT_Q8_0 && n == 1 && nu >= 128) return m >= 8192 ? Cfg{64, 1, 4, 4} : Cfg{32, 1, 4, 4};
    if (fmt == Q4_FMT_Q2_K && nu >= 128)
        return (n == 1 && nu >= 256) || (n >= 6 && nu < 256) ? Cfg{32, 1, 8, 2} : Cfg{32, 2, 4, 2};
    if (fmt == Q4_FMT_Q1_0 && n == 1 && nu <= 32 && m >= 16384) return Cfg{8, 2, 1, 8};
    if (fmt == Q4_FMT_Q4_0 || fmt == Q4_FMT_Q8_0 || fmt == Q4_FMT_Q1_0) {
        if (n == 1) {
            if (nu <= 32) return m >= 16384 ? Cfg{8, 1, 1, 8} : Cfg{32, 2, 1, 8};
            if (nu < 128) return Cfg{64, 1, 4, 4};
            return Cfg{32, 2, 4, 2};
        }
        if (nu > 32 && nu < 128) return Cfg{64, 1, 4, 4};
        if (n >= 6 && nu >= 128 && nu < 256) return Cfg{32, 1, 8, 2};
        return Cfg{32, 2, 4, 2};
    }
    if (nu > 32 && nu < 128) return Cfg{64, 1, 4, 4};
    if (nu <= 32) return n <= 2 ? Cfg{16, 1, 1, 8} : n >= 5 ? Cfg{32, 2, 4, 2} : Cfg{16, 1, 4, 4};
    if (nu >= 256) return Cfg{32, 1, 8, 2};
    if (n == 1) return m >= 8192 ? Cfg{32, 1, 8, 1} : Cfg{16, 1, 4, 4};
    return Cfg{32, 1, 8, 2};
}

// The gated product's geometry: the plain product's choice for the stacked
// 2m-row matrix, moved to a gated geometry (two row slots per lane) with the
// same lanes per row, so each gate and up row is summed exactly as the plain
// product sums it, and one-wave groups only where the plain choice has them.
// (Eight lanes per row, the plain choice for very tall short-row products,
// becomes sixteen.) 8-wave plain choices at several tokens keep their 8-wave
// groups: with the whole row's activations in the opt-in LDS, a 4-wave group
// would leave one group of 4 waves per CU.
Cfg choose_tiled(int fmt, int64_t m, int64_t k, int64_t n, int cus);

Cfg choose_glu(int fmt, int64_t m, int64_t k, int64_t n, int cus)
{
    // The matrix-core kernel where the plain product of the stacked matrix
    // would take it and the row fits its gated form (16 super-blocks).
    if (use_matrix(fmt, 2 * m, k, n) && k <= 4096) {
        Cfg c{0, 0, 0, 1};
        c.matrix = true;
        return c;
    }
    const Cfg c = choose_tiled(fmt, 2 * m, k, n, cus);
    const bool one_wave = c.waves == 1;
    if (c.lpr <= 16) return one_wave ? Cfg{16, 2, 1, 8} : Cfg{16, 2, 4, 4};
    if (c.lpr == 32) {
        if (one_wave) return Cfg{32, 2, 1, 8};
        if (c.waves == 8 && n >= 2) return Cfg{32, 2, 8, 2};
        return Cfg{32, 2, 4, 2};
    }
    return Cfg{64, 2, 4, 4};
}

int dispatch(int fmt, const Cfg &c, const void *w, const float *x, float *y, int64_t m, int64_t k, int64_t n,
             void *stream, int cus, bool glu = false)
{
    const auto *wb = static_cast<const uint8_t *>(w);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int mi = static_cast<int>(m), ki = static_cast<int>(k);
    if (c.matrix) {
        // The matrix-core kernel: Q4_K, plain or gated.
        if (fmt != Q4_FMT_Q4_K) return Q4_EUNSUPPORTED;
        return dispatch_mfma(wb, x, y, mi, ki, static_cast<int>(n), s, cus, c.groups_per_cu, glu);
    }
    if (c.depth > 0) {
        // The streaming kernel: one token, plain product, the whole row staged.
        if (glu || n != 1 || k / kUnitWeights > kStreamMaxUnits) return Q4_EUNSUPPORTED;
        switch (fmt) {
        case Q4_FMT_Q4_0: return dispatch_stream<FmtQ4_0>(c, wb, x, y, mi, ki, s, cus);
        case Q4_FMT_Q8_0: return dispatch_stream<FmtQ8_0>(c, wb, x, y, mi, ki, s, cus);
        case Q4_FMT_Q1_0: return dispatch_stream<FmtQ1_0>(c, wb, x, y, mi, ki, s, cus);
        case Q4_FMT_Q2_K: return dispatch_stream<FmtQ2_K>(c, wb, x, y, mi, ki, s, cus);
        default: return dispatch_stream<FmtQ4_K>(c, wb, x, y, mi, ki, s, cus);
        }
    }
#define Q4_N_CASE(F, NN)                                                            \
    case NN:                                                                        \
        return glu ? dispatch_glu_cfg<F, NN>(c, wb, x, y, mi, ki, s, cus)           \
                   : dispatch_cfg<F, NN>(c, wb, x, y, mi, ki, s, cus);
    if (fmt == Q4_FMT_Q4_0) {
        switch (n) {
            Q4_N_CASE(FmtQ4_0, 1) Q4_N_CASE(FmtQ4_0, 2) Q4_N_CASE(FmtQ4_0, 3) Q4_N_CASE(FmtQ4_0, 4)
            Q4_N_CASE(FmtQ4_0, 5) Q4_N_CASE(FmtQ4_0, 6) Q4_N_CASE(FmtQ4_0, 7) Q4_N_CASE(FmtQ4_0, 8)
        default: return Q4_EUNSUPPORTED;
        }
    }
    if (fmt == Q4_FMT_Q8_0) {
        switch (n) {
            Q4_N_CASE(FmtQ8_0, 1) Q4_N_CASE(FmtQ8_0, 2) Q4_N_CASE(FmtQ8_0, 3) Q4_N_CASE(FmtQ8_0, 4)
            Q4_N_CASE(FmtQ8_0, 5) Q4_N_CASE(FmtQ8_0, 6) Q4_N_CASE(FmtQ8_0, 7) Q4_N_CASE(FmtQ8_0, 8)
        default: return Q4_EUNSUPPORTED;
        }
    }
    if (fmt == Q4_FMT_Q1_0) {
        switch (n) {
            Q4_N_CASE(FmtQ1_0, 1) Q4_N_CASE(FmtQ1_0, 2) Q4_N_CASE(FmtQ1_0, 3) Q4_N_CASE(FmtQ1_0, 4)
            Q4_N_CASE(FmtQ1_0, 5) Q4_N_CASE(FmtQ1_0, 6) Q4_N_CASE(FmtQ1_0, 7) Q4_N_CASE(FmtQ1_0, 8)
        default: return Q4_EUNSUPPORTED;
        }
    }
    if (fmt == Q4_FMT_Q2_K) {
        switch (n) {
            Q4_N_CASE(FmtQ2_K, 1) Q4_N_CASE(FmtQ2_K, 2) Q4_N_CASE(FmtQ2_K, 3) Q4_N_CASE(FmtQ2_K, 4)
            Q4_N_CASE(FmtQ2_K, 5) Q4_N_CASE(FmtQ2_K, 6) Q4_N_CASE(FmtQ2_K, 7) Q4_N_CASE(FmtQ2_K, 8)
        default: return Q4_EUNSUPPORTED;
        }
    }
    switch (n) {
        Q4_N_CASE(FmtQ4_K, 1) Q4_N_CASE(FmtQ4_K, 2) Q4_N_CASE(FmtQ4_K, 3) Q4_N_CASE(FmtQ4_K, 4)
        Q4_N_CASE(FmtQ4_K, 5) Q4_N_CASE(FmtQ4_K, 6) Q4_N_CASE(FmtQ4_K, 7) Q4_N_CASE(FmtQ4_K, 8)
    default: return Q4_EUNSUPPORTED;
    }
#undef Q4_N_CASE
}

}  // namespace gemv

int launch_gemv(int fmt, const void *w, const float *x, float *y, int64_t m, int64_t k, int64_t n, void *stream)
{
    const int cus = device_cus();
    if (cus <= 0) return Q4_EHIP;
    return gemv::dispatch(fmt, gemv::choose(fmt, m, k, n, cus), w, x, y, m, k, n, stream, cus);
}

int launch_gemv_glu(int fmt, const void *w, const float *x, float *y, int64_t m, int64_t k, int64_t n, void *stream)
{
    const int cus = device_cus();
    if (cus <= 0) return Q4_EHIP;
    return gemv::dispatch(fmt, gemv::choose_glu(fmt, m, k, n, cus), w, x, y, m, k, n, stream, cus, true);
}

int launch_gemv_addnorm(int fmt, const void *w, const float *x, const Prologue &pro, float *y, int64_t m, int64_t k,
                        bool glu, void *stream, const q4_gemv_tuning *tuning)
{
    const int cus = device_cus();
    if (cus <= 0) return Q4_EHIP;
    const auto *wb = static_cast<const uint8_t *>(w);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int mi = static_cast<int>(m), ki = static_cast<int>(k);
    // The plain form takes the streaming kernel wherever the plain one-token
    // product does (the library's choice, not a tuned geometry).
    if (!glu && !tuning) {
        const gemv::Cfg cs = gemv::choose(fmt, m, k, 1, cus);
        if (cs.depth && !cs.matrix) {
            switch (fmt) {
            case Q4_FMT_Q4_0: return gemv::dispatch_stream_norm<gemv::FmtQ4_0>(cs, wb, x, y, mi, ki, s, cus, pro);
            case Q4_FMT_Q8_0: return gemv::dispatch_stream_norm<gemv::FmtQ8_0>(cs, wb, x, y, mi, ki, s, cus, pro);
            case Q4_FMT_Q1_0: return gemv::dispatch_stream_norm<gemv::FmtQ1_0>(cs, wb, x, y, mi, ki, s, cus, pro);
            case Q4_FMT_Q2_K: return gemv::dispatch_stream_norm<gemv::FmtQ2_K>(cs, wb, x, y, mi, ki, s, cus, pro);
            default: return gemv::dispatch_stream_norm<gemv::FmtQ4_K>(cs, wb, x, y, mi, ki, s, cus, pro);
            }
        }
    }
    gemv::Cfg c = glu ? gemv::choose_glu(fmt, m, k, 1, cus) : gemv::choose_tiled(fmt, m, k, 1, cus);
    // The fused norm stages three vectors (x, delta, gain) per workgroup, so
    // short-row gated products take 16 lanes per row in their one-wave groups
    // (twice the rows per group, half the groups staging): 3.7 against 4.9 us
    // at 960 -> 2 x 2560 on gfx950.
    if (glu && c.waves == 1 && c.lpr == 32) c.lpr = 16;
    if (tuning) {
        if (tuning->lanes_per_row) c.lpr = tuning->lanes_per_row;
        if (tuning->rows_per_lane) c.r = tuning->rows_per_lane;
        if (tuning->waves_per_group) c.waves = tuning->waves_per_group;
        if (tuning->groups_per_cu) c.groups_per_cu = tuning->groups_per_cu;
    }
    switch (fmt) {
    case Q4_FMT_Q4_0: return gemv::dispatch_norm_cfg<gemv::FmtQ4_0>(c, wb, x, y, mi, ki, s, cus, glu, pro);
    case Q4_FMT_Q8_0: return gemv::dispatch_norm_cfg<gemv::FmtQ8_0>(c, wb, x, y, mi, ki, s, cus, glu, pro);
    case Q4_FMT_Q2_K: return gemv::dispatch_norm_cfg<gemv::FmtQ2_K>(c, wb, x, y, mi, ki, s, cus, glu, pro);
    case Q4_FMT_Q1_0: return gemv::dispatch_norm_cfg<gemv::FmtQ1_0>(c, wb, x, y, mi, ki, s, cus, glu, pro);
    default: return gemv::dispatch_norm_cfg<gemv::FmtQ4_K>(c, wb, x, y, mi, ki, s, cus, glu, pro);
    }
}

namespace {
// [a, a + an) and [b, b + bn) (float elements) share memory.
bool overlaps(const float *a, int64_t an, const float *b, int64_t bn)
{
    const auto ia = reinterpret_cast<uintptr_t>(a), ib = reinterpret_cast<uintptr_t>(b);
    return ia < ib + 4 * static_cast<uintptr_t>(bn) && ib < ia + 4 * static_cast<uintptr_t>(an);
}
}  // namespace

int check_addnorm_args(int fmt, const void *w, const float *x, const Prologue &pro, const float *y, int64_t m,
                       int64_t k, bool glu)
{
    int st = glu ? check_glu_args(fmt, w, x, y, m, k, 1) : check_product_args(fmt, w, x, y, m, k, 1, 1);
    if (st != Q4_OK) return st;
    if (!(pro.eps >= 0.0f) || pro.eps == __builtin_huge_valf()) return Q4_EINVAL;
    if (k / kUnitWeights > kNormMaxUnits) return Q4_EUNSUPPORTED;
    if (m == 0) return Q4_OK;
    if (!pro.gain) return Q4_EINVAL;
    // The residual and the gain are read as 16-byte vectors.
    if ((reinterpret_cast<uintptr_t>(pro.gain) & 15) || (reinterpret_cast<uintptr_t>(pro.delta) & 15) ||
        (reinterpret_cast<uintptr_t>(pro.x_out) & 15))
        return Q4_EALIGN;
    // x_out is written while every workgroup reads x and delta, and y while
    // one workgroup writes x_out.
    if (pro.x_out && (overlaps(pro.x_out, k, x, k) || (pro.delta && overlaps(pro.x_out, k, pro.delta, k)) ||
                      overlaps(pro.x_out, k, y, m)))
        return Q4_EINVAL;
    return Q4_OK;
}

int check_glu_args(int fmt, const void *w, const void *x, const float *y, int64_t m, int64_t k, int64_t n)
{
    if (m < 0) return Q4_EINVAL;
    if (m >= (1LL << 29)) return Q4_EUNSUPPORTED;
    // The weights are a (2m) x k matrix; the output is n x m (within the
    // stacked matrix's own n x 2m bound).
    return check_product_args(fmt, w, x, y, 2 * m, k, n, 8);
}

int check_product_args(int fmt, const void *w, const void *x, const float *y, int64_t m, int64_t k, int64_t n,
                       int64_t n_max)
{
    if (fmt != Q4_FMT_Q4_0 && fmt != Q4_FMT_Q4_K && fmt != Q4_FMT_Q8_0 && fmt != Q4_FMT_Q2_K && fmt != Q4_FMT_Q1_0)
        return Q4_EUNSUPPORTED;
    const int64_t blk = fmt == Q4_FMT_Q4_K || fmt == Q4_FMT_Q2_K ? 256 : 32;
    if (m < 0 || k <= 0 || k % blk != 0 || n < 0) return Q4_EINVAL;
    if (n > n_max) return Q4_EUNSUPPORTED;
    if (m == 0 || n == 0) return Q4_OK;
    if (!w || !x || !y) return Q4_EINVAL;
    // 32-bit byte offsets inside the kernels: weights, x and y each < 2 GiB
    // (offsets from 2^31 up serve as the kernels' no-fetch lane offset).
    const uint64_t wbytes = static_cast<uint64_t>(q4_weight_bytes(fmt, m, k));
    if (wbytes >= (1ull << 31) || static_cast<uint64_t>(n) * k * 4 >= (1ull << 31) ||
        static_cast<uint64_t>(n) * m * 4 >= (1ull << 31) || m >= (1LL << 30))
        return Q4_EUNSUPPORTED;
    // The weights' 16-byte groups sit on 16-byte boundaries of the buffer.
    // x is read with 16-byte loads, which gfx950 serves at any 4-byte
    // alignment (its memory accesses are not alignment-checked beyond the
    // dword); y is written per element.
    if ((reinterpret_cast<uintptr_t>(w) & 15) || (reinterpret_cast<uintptr_t>(x) & 3) ||
        (reinterpret_cast<uintptr_t>(y) & 3))
        return Q4_EALIGN;
    return Q4_OK;
}

}  // namespace q4

extern "C" const char *q4_last_hip_error(void)
{
    return hipGetErrorName(q4::last_hip_error);
}

extern "C" int q4_gemv(int fmt, const void *w, const float *x, float *y, int64_t m, int64_t k, int64_t n,
                       void *hip_stream)
{
    const int st = q4::check_product_args(fmt, w, x, y, m, k, n, 8);
    if (st != Q4_OK) return st;
    if (m == 0 || n == 0) return Q4_OK;
    return q4::launch_gemv(fmt, w, x, y, m, k, n, hip_stream);
}

extern "C" int q4_gemv_glu(int fmt, const void *w, const float *x, float *y, int64_t m, int64_t k, int64_t n,
                           void *hip_stream)
{
    const int st = q4::check_glu_args(fmt, w, x, y, m, k, n);
    if (st != Q4_OK) return st;
    if (m == 0 || n == 0) return Q4_OK;
    return q4::launch_gemv_glu(fmt, w, x, y, m, k, n, hip_stream);
}

namespace {
int addnorm_entry(int fmt, const void *w, const float *x, const float *delta, const float *gain, float eps,
                  float *x_out, float *y, int64_t m, int64_t k, int epilogue, const q4_gemv_tuning *tuning,
                  void *hip_stream)
{
    if (epilogue != Q4_EPILOGUE_NONE && epilogue != Q4_EPILOGUE_SILU_MUL) return Q4_EINVAL;
    const bool glu = epilogue == Q4_EPILOGUE_SILU_MUL;
    q4::Prologue pro;
    pro.delta = delta;
    pro.gain = gain;
    pro.x_out = x_out;
    pro.eps = eps;
    const int st = q4::check_addnorm_args(fmt, w, x, pro, y, m, k, glu);
    if (st != Q4_OK) return st;
    if (m == 0) return Q4_OK;
    return q4::launch_gemv_addnorm(fmt, w, x, pro, y, m, k, glu, hip_stream, tuning);
}
}  // namespace

extern "C" int q4_gemv_addnorm(int fmt, const void *w, const float *x, const float *delta, const float *gain,
                               float eps, float *x_out, float *y, int64_t m, int64_t k, int epilogue,
                               void *hip_stream)
{
    return addnorm_entry(fmt, w, x, delta, gain, eps, x_out, y, m, k, epilogue, nullptr, hip_stream);
}

extern "C" int q4_gemv_addnorm_tuned(int fmt, const void *w, const float *x, const float *delta, const float *gain,
                                     float eps, float *x_out, float *y, int64_t m, int64_t k, int epilogue,
                                     const q4_gemv_tuning *tuning, void *hip_stream)
{
    if (!tuning) return Q4_EINVAL;
    if (tuning->lanes_per_row < 0 || tuning->rows_per_lane < 0 || tuning->waves_per_group < 0 ||
        tuning->groups_per_cu < 0 || tuning->groups_per_cu > 64 || tuning->depth < 0 || tuning->kernel < 0 ||
        tuning->kernel > Q4_GEMV_KERNEL_MATRIX)
        return Q4_EINVAL;
    // The fused norm runs on the tiled kernel only.
    if (tuning->kernel == Q4_GEMV_KERNEL_STREAM || tuning->kernel == Q4_GEMV_KERNEL_MATRIX) return Q4_EUNSUPPORTED;
    return addnorm_entry(fmt, w, x, delta, gain, eps, x_out, y, m, k, epilogue, tuning, hip_stream);
}

extern "C" int q4_gemv_tuned(int fmt, const void *w, const float *x, float *y, int64_t m, int64_t k, int64_t n,
                             const q4_gemv_tuning *tuning, void *hip_stream)
{
    int st = q4::check_product_args(fmt, w, x, y, m, k, n, 8);
    if (st != Q4_OK) return st;
    if (!tuning) return Q4_EINVAL;
    if (tuning->lanes_per_row < 0 || tuning->rows_per_lane < 0 || tuning->waves_per_group < 0 ||
        tuning->groups_per_cu < 0 || tuning->groups_per_cu > 64 || tuning->depth < 0 || tuning->kernel < 0 ||
        tuning->kernel > Q4_GEMV_KERNEL_MATRIX)
        return Q4_EINVAL;
    if (tuning->kernel == Q4_GEMV_KERNEL_STREAM && n > 1) return Q4_EUNSUPPORTED;
    // The matrix-core kernel: Q4_K only, and of the geometry fields only
    // groups_per_cu applies.
    if (tuning->kernel == Q4_GEMV_KERNEL_MATRIX &&
        (fmt != Q4_FMT_Q4_K || tuning->lanes_per_row || tuning->rows_per_lane || tuning->waves_per_group ||
         tuning->depth))
        return Q4_EUNSUPPORTED;
    if (m == 0 || n == 0) return Q4_OK;
    const int cus = q4::device_cus();
    if (cus <= 0) return Q4_EHIP;
    // The kernel: the one asked for; with Q4_GEMV_KERNEL_AUTO the tiled
    // kernel when a tiled geometry field is given, else the library's choice.
    const bool geometry = tuning->lanes_per_row || tuning->rows_per_lane || tuning->waves_per_group ||
                          tuning->groups_per_cu;
    q4::gemv::Cfg c = q4::gemv::choose(fmt, m, k, n, cus);
    if (tuning->kernel == Q4_GEMV_KERNEL_TILED || (tuning->kernel == Q4_GEMV_KERNEL_AUTO && geometry)) {
        c = q4::gemv::choose_tiled(fmt, m, k, n, cus);
    } else if (tuning->kernel == Q4_GEMV_KERNEL_STREAM && c.depth == 0) {
        c = q4::gemv::choose_stream(fmt, m, k, cus);
    } else if (tuning->kernel == Q4_GEMV_KERNEL_MATRIX) {
        c = q4::gemv::Cfg{0, 0, 0, 1};
        c.matrix = true;
    }
    if (tuning->lanes_per_row) c.lpr = tuning->lanes_per_row;
    if (tuning->rows_per_lane) c.r = tuning->rows_per_lane;
    if (tuning->waves_per_group) c.waves = tuning->waves_per_group;
    if (tuning->groups_per_cu) c.groups_per_cu = tuning->groups_per_cu;
    if (tuning->depth && c.depth) c.depth = tuning->depth;
    return q4::gemv::dispatch(fmt, c, w, x, y, m, k, n, hip_stream, cus);
}
