// One-token decode product y = W_hat x on gfx950, streaming form: every
// workgroup owns one contiguous range of rows, stages x once, and keeps up to
// D weight loads per lane in flight from its first instruction to its last.
//
// Why a second kernel for one token: a one-token product moves each weight
// byte once and does ~1.6 VALU operations per weight (Llamas on the Web,
// technical summary, Methodology section 3: dequantization in registers), so
// on MI355X the weight stream and the VALU work are of the same order and
// must overlap from the start of the launch. The tiled kernel of
// q4_gemv_kernel.h stages x per workgroup with only one weight batch in
// flight, and its weight stream starts when the staging ends. Here:
//   * one workgroup per compute unit (by default), so x is converted once per
//     CU, split over all its waves;
//   * the workgroup's rows are one contiguous range; wave v takes the row
//     groups v, v + WAVES, ... of SUBS = 64/LPR rows each; a row group is
//     streamed as ceil(nu/LPR) slots of one 32-weight unit per lane;
//   * the first D slots of every wave are requested before x is waited for,
//     and each computed slot frees its registers for the load D slots ahead;
//     no load is issued for a slot that does not exist (past the wave's last
//     slot, or a staging slot past the row's end): on gfx950 such a load
//     fetches nothing but still takes the CU's address unit a pass over 64
//     lanes (about 16 cycles for a 16-byte load), and at these sizes those
//     passes, not HBM, decided the time;
//   * the per-format decode (load and accumulate) is the tiled kernel's
//     policy, with one row per lane (R = 1) and one token;
//   * NORM: the fused residual add + RMSNorm prologue of q4_gemv_addnorm
//     (the staging forms v = x + delta, stages v * gain, sums v^2, and
//     workgroup 0 writes v out; each reduced row is scaled by
//     1/sqrt(mean(v^2) + eps), as in the tiled kernel).
#pragma once

#include <utility>

#include "q4_gemv_kernel.h"

namespace q4 {
namespace gemv {

// fn(std::integral_constant<int, v>) for the run-time value v in Is...: a
// register array indexed through it stays in registers.
template <int... Is, class Fn>
__device__ __forceinline__ void static_switch(int v, std::integer_sequence<int, Is...>, Fn &&fn)
{
    ((v == Is ? (fn(std::integral_constant<int, Is>{}), 0) : 0), ...);
}

// Activation items per thread per staging round (one round covers rows of up
// to 1536 (one wave) .. 2048 (16 waves) items of 8 activations).
template <int WAVES>
constexpr int kStreamStageRound = WAVES == 1 ? 4 : WAVES <= 4 ? 6 : WAVES <= 8 ? 3 : 2;

template <class F, int LPR, int WAVES, int D, bool LO, bool NORM = false>
__global__ __launch_bounds__(64 * WAVES) void stream_kernel(const uint8_t *__restrict__ w, uint32_t wbytes,
                                                            const float *__restrict__ x, float *__restrict__ y,
                                                            int M, int K, int rows_per_group, Prologue pro)
{
    constexpr int SUBS = 64 / LPR;
    constexpr int NT = 64 * WAVES;
    constexpr int NBUF = D + 1;
    extern __shared__ u32x4 lds[];
    const int nu = K >> 5;
    u32x4 *xs = lds;

    const int tid = threadIdx.x;
    const int wave = static_cast<int>(uniform(static_cast<uint32_t>(tid) >> 6));
    const int lane = tid & 63;
    const int sub = lane / LPR;
    const int li = lane % LPR;
    const int row0 = static_cast<int>(blockIdx.x) * rows_per_group;
    const int row_end = M - row0 < rows_per_group ? M : row0 + rows_per_group;
    const int slots = (nu + LPR - 1) / LPR;                 // slots per row group
    const int groups = (row_end - row0 + SUBS - 1) / SUBS;  // row groups of this workgroup
    const int mine = groups > wave ? (groups - wave + WAVES - 1) / WAVES : 0;
    const int total = mine * slots;                         // this wave's stream positions
    const uint32_t scale_plane = F::scale_plane(static_cast<uint64_t>(M), static_cast<uint64_t>(K));
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, static_cast<uint32_t>(K) * 4u);
    const __amdgpu_buffer_rsrc_t yr = make_rsrc(y, static_cast<uint32_t>(M) * 4u);
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(w, wbytes);

    using Regs = typename F::Regs;
    Regs buf[NBUF][1];
    // Next position to load: row group l_rg (of the workgroup), slot l_s.
    int lp = 0, l_rg = wave, l_s = 0;
    auto load_next = [&](Regs(&g)[1]) {
        const bool valid = lp < total;
        const int first = row0 + l_rg * SUBS;
        const bool live = valid && first + sub < row_end && l_s * LPR + li < nu;
        F::load(g[0], wr, scale_plane, static_cast<uint32_t>(nu),
                static_cast<uint32_t>(valid ? first : row0), static_cast<uint32_t>(sub), static_cast<uint32_t>(li),
                static_cast<uint32_t>(l_s * LPR), 0u, live);
        ++lp;
        if (++l_s == slots) {
            l_s = 0;
            l_rg += WAVES;
        }
    };
    float acc[1][1] = {{0.0f}};
    int cp = 0, c_rg = wave, c_s = 0;
    float rn = 1.0f;  // NORM: 1/rms of the staged row
    // Compute one position; at the end of a row group reduce it and store.
    // The store is issued at every position (dropped by its out-of-range
    // offset except at a row group's end) so that the compiler's wait counts
    // stay exact across the unrolled ring (stores share the loads' counter).
    auto compute_next = [&](const Regs(&g)[1]) {
        const int ul = c_s * LPR + li;
        if (ul < nu) F::template accumulate<1, 1, LO>(g, xs, ul, nu, static_cast<uint32_t>(ul), acc);
        const bool end = c_s == slots - 1;
        const int row = row0 + c_rg * SUBS + sub;
        float v = 0.0f;
        if (end) v = row_reduce<LPR>(acc[0][0]) * rn;
        const bool live = end && li == 0 && row < row_end && cp < total;
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), yr,
                                              live ? static_cast<uint32_t>(row) * 4u : kNoFetch, 0, 0);
        if (end) acc[0][0] = 0.0f;
        ++cp;
        if (++c_s == slots) {
            c_s = 0;
            c_rg += WAVES;
        }
    };

    NormIo nio{xr, xr, xr, 0.0f};
    if constexpr (NORM) {
        const uint32_t kb = static_cast<uint32_t>(K) * 4u;
        nio.delta = make_rsrc(pro.delta, pro.delta ? kb : 0u);
        nio.gain = make_rsrc(pro.gain, kb);
        nio.out = make_rsrc(pro.x_out, pro.x_out && blockIdx.x == 0 ? kb : 0u);
    }
    auto issue = [&]() {
#pragma unroll
        for (int p = 0; p < D; p++) load_next(buf[p]);
    };
    stage<F, 1, NT, kStreamStageRound<WAVES>, LO, NORM, decltype(issue), true>(xr, K, 0, nu, nu, xs, tid, nio,
                                                                             issue);
    // NORM: one sum of squares per wave, after the staged row in LDS.
    [[maybe_unused]] float *wave_ssq = reinterpret_cast<float *>(lds + kLdsSlots * nu);
    if constexpr (NORM) {
        const float sq = row_reduce<64>(nio.ssq);
        if (lane == 0) wave_ssq[wave] = sq;
    }
    wg_sync<WAVES>();
    if constexpr (NORM) {
        // Every workgroup sums the same items in the same order, so every
        // row sees the same factor.
        float sq = 0.0f;
#pragma unroll
        for (int v = 0; v < WAVES; v++) sq += wave_ssq[v];
        rn = 1.0f / __builtin_sqrtf(sq / static_cast<float>(K) + pro.eps);
    }
    if (total == 0) return;  // uniform across the wave; no barrier follows
    // Steady state: the exit is checked before each load, so every load
    // issued here fetches a real slot (a load that fetches nothing still
    // costs the address unit a pass over 64 lanes). The last D positions are
    // computed by a drain entered at the ring phase where the loads ran out,
    // so no register buffer is ever indexed at run time.
    int phase = 0;
    for (;;) {
#pragma unroll
        for (int p = 0; p < NBUF; p++) {
            if (lp >= total) {
                phase = p;
                goto drain;
            }
            load_next(buf[(p + D) % NBUF]);
            compute_next(buf[p]);
        }
    }
drain:
    static_switch(phase, std::make_integer_sequence<int, NBUF>{}, [&](auto pc) {
        constexpr int P = decltype(pc)::value;
#pragma unroll
        for (int i = 0; i < D; i++)
            if (cp < total) compute_next(buf[(P + i) % NBUF]);
    });
}

// Launch: groups_per_cu workgroups per compute unit over the rows, each a
// contiguous range of a multiple of SUBS rows. m is the number of rows.
template <class F, int LPR, int WAVES, int D, bool NORM = false>
int launch_stream(const uint8_t *w, const float *x, float *y, int m, int k, hipStream_t stream, int cus,
                  int groups_per_cu, const Prologue &pro = Prologue{})
{
    constexpr int SUBS = 64 / LPR;
    const int nu = k / kUnitWeights;
    // The staged row, plus (NORM) one float per wave for the sums of squares.
    const size_t lds = static_cast<size_t>(nu) * kLdsBytesPerUnit + (NORM ? 16u * ((WAVES + 3) / 4) : 0u);
    if (lds > static_cast<size_t>(kMaxLdsBytes)) {
        const int optin = device_lds_optin();
        if (optin <= 0 || lds > static_cast<size_t>(optin)) return Q4_EUNSUPPORTED;
        static std::atomic<int> opted[64];
        int dev = 0;
        if (hip_status(hipGetDevice(&dev)) != Q4_OK) return Q4_EHIP;
        if (dev < 0 || dev >= 64) return Q4_EUNSUPPORTED;
        if (!opted[dev].load(std::memory_order_acquire)) {
            int st = hip_status(hipFuncSetAttribute(
                reinterpret_cast<const void *>(&stream_kernel<F, LPR, WAVES, D, true, NORM>),
                hipFuncAttributeMaxDynamicSharedMemorySize, optin));
            if (st == Q4_OK)
                st = hip_status(hipFuncSetAttribute(
                    reinterpret_cast<const void *>(&stream_kernel<F, LPR, WAVES, D, false, NORM>),
                    hipFuncAttributeMaxDynamicSharedMemorySize, optin));
            if (st != Q4_OK) return st;
            opted[dev].store(1, std::memory_order_release);
        }
    }
    const long long target = static_cast<long long>(cus) * (groups_per_cu > 0 ? groups_per_cu : 1);
    long long rpg = (m + target - 1) / target;
    rpg = (rpg + SUBS - 1) / SUBS * SUBS;
    const unsigned grid = static_cast<unsigned>((m + rpg - 1) / rpg);
    const uint32_t wbytes = static_cast<uint32_t>(q4_weight_bytes(F::kFormat, m, k));
    // Activations as hi + lo fp16 pairs for matrices of fewer than kLoRowLimit
    // rows, as single fp16 values for taller ones (as the tiled kernel).
    if (m < kLoRowLimit)
        hipLaunchKernelGGL((stream_kernel<F, LPR, WAVES, D, true, NORM>), dim3(grid), dim3(64 * WAVES), lds, stream, w,
                           wbytes, x, y, m, k, static_cast<int>(rpg), pro);
    else
        hipLaunchKernelGGL((stream_kernel<F, LPR, WAVES, D, false, NORM>), dim3(grid), dim3(64 * WAVES), lds, stream,
                           w, wbytes, x, y, m, k, static_cast<int>(rpg), pro);
    return hip_status(hipGetLastError());
}

}  // namespace gemv
}  // namespace q4
