// Internal declarations shared by the host launchers of the library.
#pragma once

#include <hip/hip_runtime_api.h>

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

// Validation of a gated decode product (weights of 2m rows, output of m).
int check_glu_args(int fmt, const void *w, const void *x, const float *y, int64_t m, int64_t k, int64_t n);

// Launch one gated decode product (arguments already validated).
int launch_gemv_glu(int fmt, const void *w, const float *x, float *y,
                    int64_t m, int64_t k, int64_t n, void *stream);

// Launch one prefill product (arguments already validated).
int launch_gemm(int fmt, const void *w, const uint16_t *x, float *y,
                int64_t m, int64_t k, int64_t n, void *stream);

// Compute units of the current device (cached per device).
int device_cus();

// Largest dynamic LDS a workgroup of the current device may opt in to, in
// bytes (cached per device; <= 0 if the runtime does not report it).
int device_lds_optin();

// Q4_OK for hipSuccess, else Q4_EHIP, after recording e as the calling
// thread's last HIP error (reported by q4_last_hip_error).
int hip_status(hipError_t e);

// The fused residual add + RMSNorm ahead of a one-token decode product:
// the input is rmsnorm(x + delta) * gain, and x + delta goes to x_out.
struct Prologue {
    const float *delta = nullptr;  // null: no residual add
    const float *gain = nullptr;
    float *x_out = nullptr;        // null: not written
    float eps = 0.0f;
};

// Longest row (in 32-weight units) the fused norm takes: the whole row is
// staged in one workgroup's LDS (144 bytes per unit, 64 KiB).
constexpr int64_t kNormMaxUnits = 455;

// Validation of a fused-norm product (one token; glu: weights of 2m rows).
int check_addnorm_args(int fmt, const void *w, const float *x, const Prologue &pro, const float *y, int64_t m,
                       int64_t k, bool glu);

// Launch one fused-norm product (arguments already validated).
int launch_gemv_addnorm(int fmt, const void *w, const float *x, const Prologue &pro, float *y, int64_t m, int64_t k,
                        bool glu, void *stream, const q4_gemv_tuning *tuning = nullptr);

namespace gemv {

// Geometry of a decode launch: the tiled kernel (depth == 0), the one-token
// streaming kernel (depth > 0: slots in flight per lane; r == 1), or the
// several-token Q4_K matrix-core kernel (matrix; only groups_per_cu applies).
struct Cfg {
    int lpr;            // lanes per row: 8, 16, 32 or 64
    int r;              // rows per lane
    int waves;          // waves per workgroup
    int groups_per_cu;  // workgroups per compute unit the grid is sized for
    int depth = 0;      // streaming kernel: weight slots in flight per lane
    bool matrix = false;
};

struct FmtQ4_0;
struct FmtQ4_K;
struct FmtQ8_0;
struct FmtQ2_K;
struct FmtQ1_0;

// Defined in the per-format instantiation units (q4_gemv_q4_*.hip).
template <class F, int N>
int dispatch_cfg(const Cfg &c, const uint8_t *w, const float *x, float *y, int m, int k, hipStream_t s, int cus);
template <class F, int N>
int dispatch_glu_cfg(const Cfg &c, const uint8_t *w, const float *x, float *y, int m, int k, hipStream_t s, int cus);
template <class F>
int dispatch_norm_cfg(const Cfg &c, const uint8_t *w, const float *x, float *y, int m, int k, hipStream_t s, int cus,
                      bool glu, const Prologue &pro);
// Defined in q4_gemv_stream.hip: the one-token streaming kernel, plain and
// with the fused residual add + RMSNorm prologue.
template <class F>
int dispatch_stream(const Cfg &c, const uint8_t *w, const float *x, float *y, int m, int k, hipStream_t s, int cus);
template <class F>
int dispatch_stream_norm(const Cfg &c, const uint8_t *w, const float *x, float *y, int m, int k, hipStream_t s,
                         int cus, const Prologue &pro);

// Defined in q4_gemv_mfma.hip: the Q4_K decode product on matrix cores, any
// token count 1..8; glu: the gated product of a 2m-row matrix (rows of at
// most 4096 weights).
int dispatch_mfma(const uint8_t *w, const float *x, float *y, int m, int k, int n, hipStream_t s, int cus,
                  int groups_per_cu, bool glu = false);

// Longest row (in 32-weight units) the streaming kernel takes: the whole row
// is staged once per workgroup in its LDS (144 bytes per unit, 64 KiB).
constexpr int64_t kStreamMaxUnits = 455;

}  // namespace gemv
}  // namespace q4
