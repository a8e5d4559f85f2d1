// Decode product y = W_hat x for 4-bit block-quantized W on gfx950 (MI355X).
//
// Method (Llamas on the Web, technical summary, Methodology section 3,
// "integrated dequantization"): for the matrix-vector product of decode, the
// quantized weights are unpacked and scaled in registers and never written
// anywhere; the format decoder is a compile-time policy (same section,
// "extensibility"), so Q4_0 and Q4_K share the kernel body.
//
// gfx950 design:
//   * Memory bound: each 32-weight unit is one 16-byte nibble load (plus a
//     2-byte scale for Q4_0, a 16-byte super-block header for Q4_K). Lanes of
//     a row read consecutive 16-byte groups, so a wave instruction moves up to
//     1 KiB of one row (rows are split over LPR lanes; 64/LPR rows per wave).
//   * No MFMA: the arithmetic intensity is ~3.6 flop/byte.
//   * VALU budget: a nibble pair is turned into an fp16 pair by one AND:
//     (w & 0x000F000F) reads as two fp16 subnormals q*2^-24, and
//     (w & 0x00F000F0) as 16q*2^-24. v_dot2c_f32_f16 multiplies them with
//     fp16 activation pairs and accumulates in fp32: 9 VALU ops per 8 weights.
//     The -8 offset (Q4_0) and the mins (Q4_K) are folded in through
//     precomputed activation sums, one per 16 elements.
//   * Activations are staged once per workgroup into LDS as fp16 pairs in the
//     order the unpack produces them, each 32-element unit scaled by a power
//     of two that puts its largest magnitude in [2^14, 2^15): the scaling is
//     exact, fp16 cannot overflow, and the unit's result is rescaled by the
//     same power of two. Per-element error is one fp16 rounding (<= 2^-12
//     relative); sums are fp32.
//   * Workgroups of one wave for short rows need no s_barrier (LDS order
//     within a wave suffices); longer rows share the staging across 4 waves.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "q4_internal.h"

namespace q4 {
namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr uint32_t kLo = 0x000F000Fu;  // low nibbles of bytes 0 and 2
constexpr uint32_t kHi = 0x00F000F0u;  // high nibbles of bytes 0 and 2
constexpr int kLdsBytesPerUnit = 80;   // 64 B of fp16 pairs + 16 B of unit metadata
constexpr int kMaxLdsBytes = 64 * 1024;

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c)
{
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b), c, false);
}

__device__ __forceinline__ uint32_t pack_h2(_Float16 lo, _Float16 hi)
{
    half2_t h = {lo, hi};
    return __builtin_bit_cast(uint32_t, h);
}

__device__ __forceinline__ float half_lo(uint32_t v)
{
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(v & 0xFFFFu)));
}

__device__ __forceinline__ float half_hi(uint32_t v)
{
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(v >> 16)));
}

// Sum of the 16 products of one dword of nibbles with its four fp16 pairs.
// Pair order in xv: (L, L+2), (H, H+2)/16, (L+1, L+3), (H+1, H+3)/16.
__device__ __forceinline__ float dot_dword(uint32_t q, u32x4 xv, float acc)
{
    const uint32_t s = q >> 8;
    acc = dot2(q & kLo, xv.x, acc);
    acc = dot2(q & kHi, xv.y, acc);
    acc = dot2(s & kLo, xv.z, acc);
    acc = dot2(s & kHi, xv.w, acc);
    return acc;
}

// ---- format policies --------------------------------------------------------
// A unit is 32 weights: 16 nibble bytes whose low nibbles are 16 consecutive
// elements starting at unit_base(u) and whose high nibbles are the 16 elements
// kHighOffset further on.

struct FmtQ4_0 {
    static constexpr int kHighOffset = 16;
    static constexpr int kBatchUnits = 4;  // units (x rows) per lane per batch: 4 x 20 B in flight
    __device__ static int unit_base(int u) { return u << 5; }

    struct Regs {
        u32x4 q;
        uint32_t d;
    };
    __device__ static void load(Regs &g, const uint8_t *__restrict__ w, uint32_t scale_plane,
                                uint32_t row, uint32_t nu, uint32_t u)
    {
        const uint32_t idx = row * nu + u;
        g.q = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(w + idx * 16u));
        g.d = *reinterpret_cast<const uint16_t *>(w + scale_plane + idx * 2u);
    }
    __device__ static void zero(Regs &g)
    {
        g.q = u32x4{0, 0, 0, 0};
        g.d = 0;
    }
    // Unit metadata: x = -8 * 2^-24 * (sum of the 32 activations, scaled
    // units), z = 2^(e+24) (unit scale times the fp16-subnormal factor).
    __device__ static f32x4 meta(float gl, float gh, int e)
    {
        return f32x4{-(gl + gh) * 0x1p-21f, 0.0f, __builtin_amdgcn_ldexpf(1.0f, e + 24), 0.0f};
    }
    template <int N, int R>
    __device__ static void accumulate(const Regs (&g)[R], const u32x4 *__restrict__ xs,
                                      const f32x4 *__restrict__ meta, int ul, int uc, uint32_t /*u*/,
                                      float (&acc)[R][N])
    {
#pragma unroll
        for (int t = 0; t < N; t++) {
            const f32x4 mt = meta[t * uc + ul];
            const u32x4 x0 = xs[(t * 4 + 0) * uc + ul];
            const u32x4 x1 = xs[(t * 4 + 1) * uc + ul];
            const u32x4 x2 = xs[(t * 4 + 2) * uc + ul];
            const u32x4 x3 = xs[(t * 4 + 3) * uc + ul];
#pragma unroll
            for (int r = 0; r < R; r++) {
                float a = mt.x;
                a = dot_dword(g[r].q.x, x0, a);
                a = dot_dword(g[r].q.y, x1, a);
                a = dot_dword(g[r].q.z, x2, a);
                a = dot_dword(g[r].q.w, x3, a);
                acc[r][t] = __builtin_fmaf(half_lo(g[r].d) * mt.z, a, acc[r][t]);
            }
        }
    }
};

struct FmtQ4_K {
    static constexpr int kHighOffset = 32;
    static constexpr int kBatchUnits = 2;  // each unit is two 16-byte loads
    // unit u = slice (u & 7) of super-block u >> 3; slice h covers the 16
    // bytes at 16h of the 128 nibble bytes: chunk c = h >> 1, half h & 1.
    __device__ static int unit_base(int u) { return ((u >> 3) << 8) + (((u & 7) >> 1) << 6) + ((u & 1) << 4); }

    struct Regs {
        u32x4 q;
        u32x4 h;
    };
    __device__ static void load(Regs &g, const uint8_t *__restrict__ w, uint32_t /*scale_plane*/,
                                uint32_t row, uint32_t nu, uint32_t u)
    {
        const uint32_t base = (row * (nu >> 3) + (u >> 3)) * 144u;
        g.h = *reinterpret_cast<const u32x4 *>(w + base);
        g.q = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(w + base + 16u + ((u & 7u) << 4)));
    }
    __device__ static void zero(Regs &g)
    {
        g.q = u32x4{0, 0, 0, 0};
        g.h = u32x4{0, 0, 0, 0};
    }
    // Unit metadata: x = sum of the 16 low-nibble activations, y = 16 x sum of
    // the 16 pre-divided high-nibble activations (both scaled units),
    // z = 2^(e+24), w = 2^e.
    __device__ static f32x4 meta(float gl, float gh, int e)
    {
        return f32x4{gl, gh, __builtin_amdgcn_ldexpf(1.0f, e + 24), __builtin_amdgcn_ldexpf(1.0f, e)};
    }
    template <int N, int R>
    __device__ static void accumulate(const Regs (&g)[R], const u32x4 *__restrict__ xs,
                                      const f32x4 *__restrict__ meta, int ul, int uc, uint32_t u,
                                      float (&acc)[R][N])
    {
        // Sub-blocks a = 2c (low nibbles) and b = 2c+1 (high nibbles), c = (u & 7) >> 1.
        // Their 6-bit fields sit in bytes 2(c&1) and 2(c&1)+1 of the S words.
        const uint32_t c = (u & 7u) >> 1;
        const uint32_t sh = (c & 1u) << 4;
        const bool upper = c >= 2;
        float sca[R], scb[R], ma[R], mb[R], fd[R], fm[R];
#pragma unroll
        for (int r = 0; r < R; r++) {
            const uint32_t s0 = g[r].h.y >> sh, s1 = g[r].h.z >> sh, s2 = g[r].h.w >> sh;
            const uint32_t sca_i = upper ? ((s2 & 15u) | (((s0 >> 6) & 3u) << 4)) : (s0 & 63u);
            const uint32_t scb_i = upper ? (((s2 >> 8) & 15u) | (((s0 >> 14) & 3u) << 4)) : ((s0 >> 8) & 63u);
            const uint32_t ma_i = upper ? (((s2 >> 4) & 15u) | (((s1 >> 6) & 3u) << 4)) : (s1 & 63u);
            const uint32_t mb_i = upper ? (((s2 >> 12) & 15u) | (((s1 >> 14) & 3u) << 4)) : ((s1 >> 8) & 63u);
            sca[r] = static_cast<float>(sca_i);
            scb[r] = static_cast<float>(scb_i);
            ma[r] = static_cast<float>(ma_i);
            mb[r] = static_cast<float>(mb_i);
            fd[r] = half_lo(g[r].h.x);
            fm[r] = half_hi(g[r].h.x);
        }
#pragma unroll
        for (int t = 0; t < N; t++) {
            const f32x4 mt = meta[t * uc + ul];
            const u32x4 x0 = xs[(t * 4 + 0) * uc + ul];
            const u32x4 x1 = xs[(t * 4 + 1) * uc + ul];
            const u32x4 x2 = xs[(t * 4 + 2) * uc + ul];
            const u32x4 x3 = xs[(t * 4 + 3) * uc + ul];
#pragma unroll
            for (int r = 0; r < R; r++) {
                float aa = 0.0f, ab = 0.0f;
                const u32x4 q = g[r].q;
                // Each dword: pairs 0 and 2 belong to sub-block a, 1 and 3 to b.
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const uint32_t qi = i == 0 ? q.x : i == 1 ? q.y : i == 2 ? q.z : q.w;
                    const u32x4 xv = i == 0 ? x0 : i == 1 ? x1 : i == 2 ? x2 : x3;
                    const uint32_t s = qi >> 8;
                    aa = dot2(qi & kLo, xv.x, aa);
                    ab = dot2(qi & kHi, xv.y, ab);
                    aa = dot2(s & kLo, xv.z, aa);
                    ab = dot2(s & kHi, xv.w, ab);
                }
                const float t1 = __builtin_fmaf(scb[r], ab, sca[r] * aa);
                const float t2 = __builtin_fmaf(mb[r], mt.y, ma[r] * mt.x);
                acc[r][t] = __builtin_fmaf(fd[r] * mt.z, t1, acc[r][t]);
                acc[r][t] = __builtin_fmaf(-fm[r] * mt.w, t2, acc[r][t]);
            }
        }
    }
};

// ---- workgroup synchronisation -----------------------------------------------

template <int WAVES>
__device__ __forceinline__ void wg_sync()
{
    if constexpr (WAVES == 1) {
        // One wave: its LDS operations complete in issue order, so only the
        // compiler must be kept from moving LDS accesses across this point.
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        __builtin_amdgcn_wave_barrier();
    } else {
        __syncthreads();
    }
}

// ---- activation staging -------------------------------------------------------
// Units [c0, c0 + nuc) of every token -> LDS. Item (t, ul, i) handles dword i
// of unit ul: activations L..L+3 (low nibbles) and H..H+3 (high nibbles),
// L = unit_base + 4i, H = L + kHighOffset. The four items of a unit are four
// consecutive lanes, which exchange their maxima and partial sums.

template <class F, int N, int NT>
__device__ __forceinline__ void stage(const float *__restrict__ x, int K, int c0, int nuc, int uc,
                                      u32x4 *__restrict__ xs, f32x4 *__restrict__ meta, int tid)
{
    const int per_tok = nuc * 4;
    for (int it = tid; it < N * per_tok; it += NT) {
        const int t = it / per_tok;
        const int rem = it - t * per_tok;
        const int ul = rem >> 2;
        const int i = rem & 3;
        const int L = F::unit_base(c0 + ul) + 4 * i;
        const int H = L + F::kHighOffset;
        const float *xt = x + static_cast<size_t>(t) * K;
        const f32x4 a = *reinterpret_cast<const f32x4 *>(xt + L);
        const f32x4 b = *reinterpret_cast<const f32x4 *>(xt + H);
        float mx = __builtin_fmaxf(__builtin_fmaxf(__builtin_fabsf(a.x), __builtin_fabsf(a.y)),
                                   __builtin_fmaxf(__builtin_fabsf(a.z), __builtin_fabsf(a.w)));
        mx = __builtin_fmaxf(mx, __builtin_fmaxf(__builtin_fmaxf(__builtin_fabsf(b.x), __builtin_fabsf(b.y)),
                                                 __builtin_fmaxf(__builtin_fabsf(b.z), __builtin_fabsf(b.w))));
        mx = __builtin_fmaxf(mx, __shfl_xor(mx, 1));
        mx = __builtin_fmaxf(mx, __shfl_xor(mx, 2));
        // Largest magnitude -> [2^14, 2^15): x_tilde = x * 2^-e.
        const int e = __builtin_amdgcn_frexp_expf(mx) - 15;
        const _Float16 l0 = static_cast<_Float16>(__builtin_amdgcn_ldexpf(a.x, -e));
        const _Float16 l1 = static_cast<_Float16>(__builtin_amdgcn_ldexpf(a.y, -e));
        const _Float16 l2 = static_cast<_Float16>(__builtin_amdgcn_ldexpf(a.z, -e));
        const _Float16 l3 = static_cast<_Float16>(__builtin_amdgcn_ldexpf(a.w, -e));
        const _Float16 h0 = static_cast<_Float16>(__builtin_amdgcn_ldexpf(b.x, -e - 4));
        const _Float16 h1 = static_cast<_Float16>(__builtin_amdgcn_ldexpf(b.y, -e - 4));
        const _Float16 h2 = static_cast<_Float16>(__builtin_amdgcn_ldexpf(b.z, -e - 4));
        const _Float16 h3 = static_cast<_Float16>(__builtin_amdgcn_ldexpf(b.w, -e - 4));
        xs[(t * 4 + i) * uc + ul] = u32x4{pack_h2(l0, l2), pack_h2(h0, h2), pack_h2(l1, l3), pack_h2(h1, h3)};
        float gl = (static_cast<float>(l0) + static_cast<float>(l1)) + (static_cast<float>(l2) + static_cast<float>(l3));
        float gh = (static_cast<float>(h0) + static_cast<float>(h1)) + (static_cast<float>(h2) + static_cast<float>(h3));
        gl += __shfl_xor(gl, 1);
        gh += __shfl_xor(gh, 1);
        gl += __shfl_xor(gl, 2);
        gh += __shfl_xor(gh, 2);
        if (i == 0) meta[t * uc + ul] = F::meta(gl, 16.0f * gh, e);
    }
}

// ---- the kernel -------------------------------------------------------------------
// Workgroup = WAVES waves; a wave covers RPW = (64/LPR)*R rows: sub-group s
// (lanes s*LPR .. s*LPR+LPR-1) handles rows row0 + s + r*(64/LPR), r < R.
// Lane li of a sub-group handles units li, li+LPR, ... of each of its rows,
// in batches of JB units per row, double-buffered. LDS holds the activations
// of uc units per token; longer rows are processed in chunks.

template <class F, int N, int LPR, int R, int WAVES, int JB>
__global__ __launch_bounds__(64 * WAVES) void gemv_kernel(const uint8_t *__restrict__ w,
                                                          const float *__restrict__ x,
                                                          float *__restrict__ y, int M, int K, int uc)
{
    constexpr int SUBS = 64 / LPR;
    constexpr int RPW = SUBS * R;
    constexpr int NT = 64 * WAVES;
    extern __shared__ u32x4 lds[];
    u32x4 *xs = lds;
    f32x4 *meta = reinterpret_cast<f32x4 *>(lds + N * 4 * uc);

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int sub = lane / LPR;
    const int li = lane % LPR;
    const int nu = K >> 5;
    const uint32_t scale_plane = static_cast<uint32_t>(static_cast<uint64_t>(M) * static_cast<uint64_t>(K) / 2u);
    const int row0 = blockIdx.x * (WAVES * RPW) + wave * RPW + sub;

    float acc[R][N];
#pragma unroll
    for (int r = 0; r < R; r++)
#pragma unroll
        for (int t = 0; t < N; t++) acc[r][t] = 0.0f;

    using Regs = typename F::Regs;

    for (int c0 = 0; c0 < nu; c0 += uc) {
        const int nuc = nu - c0 < uc ? nu - c0 : uc;
        const int jc = (nuc + LPR - 1) / LPR;  // unit slots per lane per row in this chunk

        auto load_batch = [&](Regs(&g)[JB][R], int j0) {
#pragma unroll
            for (int jj = 0; jj < JB; jj++) {
                const int ul = li + (j0 + jj) * LPR;
#pragma unroll
                for (int r = 0; r < R; r++) {
                    const int row = row0 + r * SUBS;
                    if (ul < nuc && row < M)
                        F::load(g[jj][r], w, scale_plane, static_cast<uint32_t>(row), static_cast<uint32_t>(nu),
                                static_cast<uint32_t>(c0 + ul));
                    else
                        F::zero(g[jj][r]);
                }
            }
        };
        auto compute_batch = [&](const Regs(&g)[JB][R], int j0) {
#pragma unroll
            for (int jj = 0; jj < JB; jj++) {
                const int ul = li + (j0 + jj) * LPR;
                if (ul < nuc) F::template accumulate<N, R>(g[jj], xs, meta, ul, uc, static_cast<uint32_t>(c0 + ul), acc);
            }
        };

        Regs ga[JB][R], gb[JB][R];
        // Weight loads go out before the activations are staged, so their HBM
        // latency overlaps the staging.
        load_batch(ga, 0);
        if (c0 > 0) wg_sync<WAVES>();
        stage<F, N, NT>(x, K, c0, nuc, uc, xs, meta, tid);
        wg_sync<WAVES>();

        for (int j0 = 0; j0 < jc; j0 += 2 * JB) {
            if (j0 + JB < jc) load_batch(gb, j0 + JB);
            compute_batch(ga, j0);
            if (j0 + JB >= jc) break;
            if (j0 + 2 * JB < jc) load_batch(ga, j0 + 2 * JB);
            compute_batch(gb, j0 + JB);
        }
    }

    // Reduce each row's partial sums over its LPR lanes and store.
#pragma unroll
    for (int r = 0; r < R; r++) {
        const int row = row0 + r * SUBS;
#pragma unroll
        for (int t = 0; t < N; t++) {
            float v = acc[r][t];
#pragma unroll
            for (int off = LPR / 2; off >= 1; off >>= 1) v += __shfl_xor(v, off);
            if (li == 0 && row < M) y[static_cast<size_t>(t) * M + row] = v;
        }
    }
}

// ---- launch configuration ---------------------------------------------------------

struct Cfg {
    int lpr, r, waves;
};

template <class F, int N, int LPR, int R, int WAVES>
int launch_one(const uint8_t *w, const float *x, float *y, int m, int k, hipStream_t stream, int cus)
{
    constexpr int JB = F::kBatchUnits / R > 0 ? F::kBatchUnits / R : 1;
    constexpr int rows_per_wg = WAVES * (64 / LPR) * R;
    (void)cus;
    const int nu = k / 32;
    int uc = nu;
    const int bytes_per_unit = N * kLdsBytesPerUnit;
    if (uc * bytes_per_unit > kMaxLdsBytes) uc = (kMaxLdsBytes / bytes_per_unit) / LPR * LPR;
    if (uc <= 0) return Q4_EUNSUPPORTED;
    const size_t lds = static_cast<size_t>(uc) * bytes_per_unit;
    const unsigned grid = static_cast<unsigned>((m + rows_per_wg - 1) / rows_per_wg);
    hipLaunchKernelGGL((gemv_kernel<F, N, LPR, R, WAVES, JB>), dim3(grid), dim3(64 * WAVES), lds, stream, w, x, y,
                       m, k, uc);
    return hipGetLastError() == hipSuccess ? Q4_OK : Q4_EHIP;
}

template <class F, int N>
int dispatch_cfg(const Cfg &c, const uint8_t *w, const float *x, float *y, int m, int k, hipStream_t s, int cus)
{
#define Q4_CFG(L, RR, WV)                                                     \
    if (c.lpr == L && c.r == RR && c.waves == WV) return launch_one<F, N, L, RR, WV>(w, x, y, m, k, s, cus);
    Q4_CFG(8, 1, 1)
    Q4_CFG(8, 2, 1)
    Q4_CFG(8, 4, 1)
    Q4_CFG(16, 1, 1)
    Q4_CFG(16, 2, 1)
    Q4_CFG(32, 1, 1)
    Q4_CFG(32, 2, 1)
    Q4_CFG(16, 1, 4)
    Q4_CFG(32, 1, 4)
    Q4_CFG(64, 1, 4)
    Q4_CFG(64, 2, 4)
#undef Q4_CFG
    return Q4_EUNSUPPORTED;
}

template <class F>
int dispatch_n(const Cfg &c, const uint8_t *w, const float *x, float *y, int m, int k, int n, hipStream_t s, int cus)
{
    switch (n) {
    case 1: return dispatch_cfg<F, 1>(c, w, x, y, m, k, s, cus);
    case 2: return dispatch_cfg<F, 2>(c, w, x, y, m, k, s, cus);
    case 3: return dispatch_cfg<F, 3>(c, w, x, y, m, k, s, cus);
    case 4: return dispatch_cfg<F, 4>(c, w, x, y, m, k, s, cus);
    case 5: return dispatch_cfg<F, 5>(c, w, x, y, m, k, s, cus);
    case 6: return dispatch_cfg<F, 6>(c, w, x, y, m, k, s, cus);
    case 7: return dispatch_cfg<F, 7>(c, w, x, y, m, k, s, cus);
    case 8: return dispatch_cfg<F, 8>(c, w, x, y, m, k, s, cus);
    default: return Q4_EUNSUPPORTED;
    }
}

}  // namespace

// Geometry choice: enough units per lane to amortise the cross-lane
// reduction, one-wave workgroups (no barrier) for short rows, and as many
// rows per lane as keeps at least two workgroups per compute unit.
Cfg choose_gemv_cfg(int64_t m, int64_t k, int64_t n, int cus)
{
    const int64_t nu = k / 32;
    int lpr = 64;
    while (lpr > 8 && nu < 2 * lpr) lpr >>= 1;
    int waves = nu <= 32 ? 1 : 4;
    if (waves == 1 && lpr > 32) lpr = 32;
    if (waves == 4 && lpr < 16) lpr = 16;
    int r = 1;
    const int64_t target = 2LL * cus;
    const int rmax = (waves == 1 && lpr == 8) ? 4 : (lpr <= 32 && waves == 1) || lpr == 64 ? 2 : 1;
    for (int cand = rmax; cand > 1; cand >>= 1) {
        const int64_t rows = static_cast<int64_t>(waves) * (64 / lpr) * cand;
        if ((m + rows - 1) / rows >= target) { r = cand; break; }
    }
    (void)n;
    return Cfg{lpr, r, waves};
}

int launch_gemv(int fmt, const void *w, const float *x, float *y, int64_t m, int64_t k, int64_t n, void *stream)
{
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) != hipSuccess) return Q4_EHIP;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return Q4_EHIP;
    const Cfg c = choose_gemv_cfg(m, k, n, cus);
    const auto *wb = static_cast<const uint8_t *>(w);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (fmt == Q4_FMT_Q4_0) return dispatch_n<FmtQ4_0>(c, wb, x, y, (int)m, (int)k, (int)n, s, cus);
    return dispatch_n<FmtQ4_K>(c, wb, x, y, (int)m, (int)k, (int)n, s, cus);
}

int check_product_args(int fmt, const void *w, const void *x, const float *y, int64_t m, int64_t k, int64_t n,
                       int64_t n_max)
{
    if (fmt != Q4_FMT_Q4_0 && fmt != Q4_FMT_Q4_K) return Q4_EUNSUPPORTED;
    const int64_t blk = fmt == Q4_FMT_Q4_0 ? 32 : 256;
    if (m < 0 || k <= 0 || k % blk != 0 || n < 0) return Q4_EINVAL;
    if (n > n_max) return Q4_EUNSUPPORTED;
    if (m == 0 || n == 0) return Q4_OK;
    if (!w || !x || !y) return Q4_EINVAL;
    // 32-bit byte offsets inside the kernels: weights < 4 GiB, x and y < 2 GiB.
    const uint64_t wbytes = static_cast<uint64_t>(q4_weight_bytes(fmt, m, k));
    if (wbytes >= (1ull << 32) || static_cast<uint64_t>(n) * k * 4 >= (1ull << 31) ||
        static_cast<uint64_t>(n) * m * 4 >= (1ull << 31) || m >= (1LL << 30))
        return Q4_EUNSUPPORTED;
    if ((reinterpret_cast<uintptr_t>(w) & 15) || (reinterpret_cast<uintptr_t>(x) & 15) ||
        (reinterpret_cast<uintptr_t>(y) & 3))
        return Q4_EALIGN;
    return Q4_OK;
}

}  // namespace q4

extern "C" int q4_gemv(int fmt, const void *w, const float *x, float *y, int64_t m, int64_t k, int64_t n,
                       void *hip_stream)
{
    int st = q4::check_product_args(fmt, w, x, y, m, k, n, 8);
    if (st != Q4_OK) return st;
    if (m == 0 || n == 0) return Q4_OK;
    return q4::launch_gemv(fmt, w, x, y, m, k, n, hip_stream);
}
