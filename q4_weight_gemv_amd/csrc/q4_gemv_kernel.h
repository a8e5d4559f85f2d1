// Decode product y = W_hat x for 4-bit block-quantized W on gfx950 (MI355X):
// device code, shared by the per-format instantiation units.
//
// Method (Llamas on the Web, technical summary, Methodology section 3,
// "integrated dequantization"): for the matrix-vector product of decode, the
// quantized weights are unpacked and scaled in registers and never written
// anywhere; the format decoder is a compile-time policy (same section,
// "extensibility"), so Q4_0, Q4_K, Q8_0, Q2_K and Q1_0 share the kernel body
// (the notes below describe the 4-bit formats; each policy states its own
// unit). The same body also serves the gated epilogue (GLU) and the fused
// residual add + RMSNorm prologue (NORM).
//
// gfx950 design:
//   * Memory bound: each 32-weight unit is one 16-byte nibble load (plus a
//     2-byte scale for Q4_0, a 16-byte super-block header for Q4_K). Lanes of
//     a row read consecutive 16-byte groups, so a wave instruction moves up to
//     1 KiB of one row (rows are split over LPR lanes; 64/LPR rows per wave).
//   * No MFMA: the arithmetic intensity is ~3.6 flop/byte.
//   * VALU budget: a nibble pair is turned into an fp16 pair by one AND:
//     (w & 0x000F000F) reads as two fp16 subnormals q*2^-24, and
//     (w & 0x00F000F0) as 16q*2^-24. One packed fp16 fma, times 1024 less
//     8*2^-14 (128*2^-14), makes them (q-8)*2^-14 (16(q-8)*2^-14), exact
//     normal fp16 values (or zero), so every product (q-8)*x is exact and a
//     zero weight contributes exactly zero. v_dot2c_f32_f16 multiplies the
//     pairs with fp16 activation pairs and accumulates in fp32. The codes
//     are moved out of the fp16 subnormal range on purpose: fed subnormal
//     operands, v_dot2c_f32_f16 on gfx950 keeps fewer bits of the products
//     and rounds them down (a measured mean error of -2^-22 of the unit's
//     term scale per 32-weight unit, the same sign for every row), while
//     with normal operands it matches a chain of IEEE fp32 fmas. Q4_K keeps
//     unsigned codes (a packed multiply by 1024) and folds its mins in
//     through precomputed activation sums, one per 16 elements (the format's
//     value is itself that difference of two terms).
//   * Activations are staged once per workgroup into LDS as fp16 pairs in the
//     order the unpack produces them, each 32-element unit scaled by a power
//     of two that puts its largest magnitude in [2^14, 2^15): the scaling is
//     exact, fp16 cannot overflow, and the unit's result is rescaled by the
//     same power of two. For products of fewer than kLoRowLimit rows each
//     scaled activation is held as an unevaluated sum hi + lo of two fp16
//     values (lo = fp16(x - hi)), about 2^-23 relative, so every product term
//     is as accurate as fp32 arithmetic (the second half costs a second dot2
//     per pair); taller products keep hi only (round to nearest: at most
//     2^-11 relative per activation, so each output is within
//     2^-11 * sum_k |w_ik x_k| plus the fp32 sums' rounding), which halves the dot
//     issues, the activation LDS reads and most of the staging work.
//   * Workgroups of one wave for short rows need no s_barrier (LDS order
//     within a wave suffices); longer rows share the staging across 4 waves.
#pragma once

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <type_traits>

#include "q4_internal.h"

namespace q4 {
namespace gemv {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr uint32_t kLo = 0x000F000Fu;  // low nibbles of bytes 0 and 2
constexpr uint32_t kHi = 0x00F000F0u;  // high nibbles of bytes 0 and 2
constexpr int kLdsBytesPerUnit = 144;  // 2 x 64 B of fp16 pairs (hi, lo) + 16 B of unit metadata
// LDS layout of the staged activations, unit-major: (token t, unit ul) owns
// nine 16-byte slots from xslot(t, ul, uc): the hi and lo fp16 pairs of
// nibble dword i at 2i and 2i + 1, the unit's metadata at 8. One address per
// unit, the slots as immediate offsets; consecutive lanes read units 144 B
// apart, which falls on distinct LDS banks for a 16-byte read.
constexpr int kLdsSlots = 9;
__device__ __forceinline__ int xslot(int t, int ul, int uc) { return (t * uc + ul) * kLdsSlots; }
constexpr int kMaxLdsBytes = 64 * 1024;
// Products with fewer rows hold activations as hi + lo fp16 pairs; taller
// ones as a single fp16 each (see launch_one).
constexpr int kLoRowLimit = 256;
// Activation items per thread per staging round: one round covers a
// 11008-long row for one token in a 4-wave group (1376 items / 256 threads).
template <int WAVES>
constexpr int kStageRound = WAVES == 1 ? 4 : 6;

// Raw buffer loads: base + voffset + soffset (+ immediate), range-checked by
// the hardware against num_records (an out-of-range load returns 0 and does
// not fault), so ragged rows and tiles need no clamps or branches.
// Descriptor word 3 for the gfx9 family: 32-bit untyped raw buffer.
constexpr int kBufferWord3 = 0x00020000;
constexpr int kNonTemporal = 2;  // cache policy bit: streamed data, not kept
// A per-lane offset past every descriptor's range (weight buffers are below
// 2 GiB): the load returns zeros and sends no request to memory. Slots past
// the end of a row and rows past M are pointed here, so every byte fetched
// from memory is a byte some lane uses.
constexpr uint32_t kNoFetch = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), static_cast<short>(0), static_cast<int>(bytes),
                                             kBufferWord3);
}

// A wave-uniform value stated as such (kept in a scalar register): the
// uniform part of a load's offset goes into the instruction's scalar offset.
// Only the per-lane offset is range-checked against the descriptor, and a
// live lane's whole offset lies inside the buffer by construction, so a lane
// pointed at kNoFetch still reads zeros without a memory request.
__device__ __forceinline__ uint32_t uniform(uint32_t v)
{
    return static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(v)));
}

template <int AUX>
__device__ __forceinline__ u32x4 load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff)
{
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, AUX));
}

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c)
{
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b), c, false);
}

__device__ __forceinline__ uint32_t pack_h2(_Float16 lo, _Float16 hi)
{
    half2_t h = {lo, hi};
    return __builtin_bit_cast(uint32_t, h);
}

// x = hi + lo (+ at most 2^-24 |x|): hi = fp16(x), lo = fp16(x - hi); the
// difference x - hi is exact in fp32.
struct Split {
    _Float16 hi, lo;
};
__device__ __forceinline__ Split split(float x)
{
    const _Float16 hi = static_cast<_Float16>(x);
    const _Float16 lo = static_cast<_Float16>(x - static_cast<float>(hi));
    return Split{hi, lo};
}

__device__ __forceinline__ float half_lo(uint32_t v)
{
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(v & 0xFFFFu)));
}

__device__ __forceinline__ float half_hi(uint32_t v)
{
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(v >> 16)));
}

// Masked code bits c*2^-24 (an fp16 subnormal pair, c < 1024) as the normal
// pair c*2^-14 - OFF*2^-14: one packed fp16 fma, exact (c*2^-14 and the
// result have at most 11 significant bits and lie in the normal range, or
// are zero). Every code below carries the factor 2^-14 (kCodeExp), which
// the unit's metadata scale removes.
constexpr int kCodeExp = 14;
template <int OFF>
__device__ __forceinline__ uint32_t code_pair(uint32_t v)
{
    const half2_t h = __builtin_bit_cast(half2_t, v);
    const _Float16 k = static_cast<_Float16>(1024.0f);
    const _Float16 o = static_cast<_Float16>(-static_cast<float>(OFF) * 0x1p-14f);
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(h, half2_t{k, k}, half2_t{o, o}));
}

// Q4_0 codes as signed normal fp16 pairs: (q-8)*2^-14 for low nibbles,
// 16(q-8)*2^-14 for high nibbles.
template <bool LO>
__device__ __forceinline__ float dot_dword(uint32_t q, u32x4 xh, u32x4 xl, float acc)
{
    const uint32_t s = q >> 8;
    const uint32_t p0 = code_pair<8>(q & kLo), p1 = code_pair<128>(q & kHi);
    const uint32_t p2 = code_pair<8>(s & kLo), p3 = code_pair<128>(s & kHi);
    acc = dot2(p0, xh.x, acc);
    acc = dot2(p1, xh.y, acc);
    acc = dot2(p2, xh.z, acc);
    acc = dot2(p3, xh.w, acc);
    if constexpr (LO) {
        acc = dot2(p0, xl.x, acc);
        acc = dot2(p1, xl.y, acc);
        acc = dot2(p2, xl.z, acc);
        acc = dot2(p3, xl.w, acc);
    }
    return acc;
}

// ---- format policies --------------------------------------------------------
// A unit is 32 weights: 16 nibble bytes whose low nibbles are 16 consecutive
// elements starting at unit_base(u) and whose high nibbles are the 16 elements
// kHighOffset further on.

struct FmtQ4_0 {
    static constexpr int kFormat = Q4_FMT_Q4_0;
    static constexpr int kHighOffset = 16;
    static constexpr int kBatchUnits = 4;  // units (x rows) per lane per batch: 4 x 20 B in flight
    __device__ static int unit_base(int u) { return u << 5; }
    __device__ static int item_base(int u, int i) { return unit_base(u) + 4 * i; }
    __device__ static uint32_t scale_plane(uint64_t rows, uint64_t k) { return static_cast<uint32_t>(rows * k / 2u); }

    struct Regs {
        u32x4 q;
        uint32_t d;
    };
    // Unit (row, u) with row = trow + rowrel and u = ubase + li + jl: its
    // 16 nibble bytes at (row*nu + u)*16, its scale at scale_plane +
    // (row*nu + u)*2. The lane part goes in the VGPR offset, the uniform part
    // (tile, chunk, batch) in the SGPR offset, jl in the immediate.
    __device__ static void load(Regs &g, __amdgpu_buffer_rsrc_t wr, uint32_t scale_plane, uint32_t nu,
                                uint32_t trow, uint32_t rowrel, uint32_t li, uint32_t ubase, uint32_t jl, bool live)
    {
        const uint32_t uni_u = uniform(trow * nu + ubase);
        const uint32_t lane_u = rowrel * nu + li + jl;
        g.q = load16<kNonTemporal>(wr, live ? lane_u * 16u : kNoFetch, uni_u * 16u);
        g.d = __builtin_amdgcn_raw_buffer_load_b16(wr, live ? lane_u * 2u : kNoFetch, scale_plane + uni_u * 2u, 0);
    }
    // Unit metadata: z = 2^(e+14) (the unit's activation scale times the
    // codes' factor 2^14).
    __device__ static f32x4 meta(float /*gl*/, float /*gh*/, int e)
    {
        return f32x4{0.0f, 0.0f, __builtin_amdgcn_ldexpf(1.0f, e + kCodeExp), 0.0f};
    }
    template <int N, int R, bool LO>
    __device__ static void accumulate(const Regs (&g)[R], const u32x4 *__restrict__ xs,
                                      int ul, int uc, uint32_t /*u*/,
                                      float (&acc)[R][N])
    {
#pragma unroll
        for (int t = 0; t < N; t++) {
            const u32x4 *xu = xs + xslot(t, ul, uc);
            const f32x4 mt = __builtin_bit_cast(f32x4, xu[8]);
            u32x4 xh[4], xl[4];
#pragma unroll
            for (int i = 0; i < 4; i++) {
                xh[i] = xu[2 * i];
                xl[i] = LO ? xu[2 * i + 1] : u32x4{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int r = 0; r < R; r++) {
                float a = 0.0f;
                a = dot_dword<LO>(g[r].q.x, xh[0], xl[0], a);
                a = dot_dword<LO>(g[r].q.y, xh[1], xl[1], a);
                a = dot_dword<LO>(g[r].q.z, xh[2], xl[2], a);
                a = dot_dword<LO>(g[r].q.w, xh[3], xl[3], a);
                acc[r][t] = __builtin_fmaf(half_lo(g[r].d) * mt.z, a, acc[r][t]);
            }
        }
    }
};

// Q8_0 codes as exact fp16 pairs: a byte permute places two code bytes
// (offset by 128, so 0..255) under the exponent byte E, and one packed add
// removes the offset. E = 0x64 gives 1024 + u (spacing 1), so adding -1152
// leaves the code q; E = 0x74 gives 16384 + 16u (spacing 16), so adding
// -18432 leaves 16q. Both exact.
template <uint32_t E, int S>
__device__ __forceinline__ uint32_t q8_pair(uint32_t u)
{
    // Bytes {S, E, S+2, E}: the codes of elements S and S+2 of the dword.
    constexpr uint32_t sel = S == 0 ? 0x04020400u : 0x04030401u;
    const half2_t h = __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(E * 0x01010101u, u, sel));
    constexpr float off = E == 0x64u ? -1152.0f : -18432.0f;
    return __builtin_bit_cast(uint32_t, h + half2_t{static_cast<_Float16>(off), static_cast<_Float16>(off)});
}

// Q8_0: a unit is one block, 32 code bytes (elements in order) and an fp16
// scale in the scale plane. The activations are staged as for Q4_0 (pairs
// (L, L+2), (H, H+2)/16, (L+1, L+3), (H+1, H+3)/16, H = L + 16), so the codes
// of the block's second half enter as 16q.
struct FmtQ8_0 {
    static constexpr int kFormat = Q4_FMT_Q8_0;
    static constexpr int kHighOffset = 16;
    static constexpr int kBatchUnits = 2;  // each unit is two 16-byte loads and a scale
    __device__ static int unit_base(int u) { return u << 5; }
    __device__ static int item_base(int u, int i) { return unit_base(u) + 4 * i; }
    __device__ static uint32_t scale_plane(uint64_t rows, uint64_t k) { return static_cast<uint32_t>(rows * k); }

    struct Regs {
        u32x4 q0, q1;  // code bytes 0..15 and 16..31
        uint32_t d;
    };
    // Unit (row, u), row = trow + rowrel, u = ubase + li + jl: its 32 code
    // bytes at (row*nu + u)*32, its scale at scale_plane + (row*nu + u)*2.
    __device__ static void load(Regs &g, __amdgpu_buffer_rsrc_t wr, uint32_t scale_plane, uint32_t nu,
                                uint32_t trow, uint32_t rowrel, uint32_t li, uint32_t ubase, uint32_t jl, bool live)
    {
        const uint32_t uni_u = uniform(trow * nu + ubase);
        const uint32_t lane_u = rowrel * nu + li + jl;
        const uint32_t off = live ? lane_u * 32u : kNoFetch;
        g.q0 = load16<kNonTemporal>(wr, off, uni_u * 32u);
        g.q1 = load16<kNonTemporal>(wr, off + 16u, uni_u * 32u);
        g.d = __builtin_amdgcn_raw_buffer_load_b16(wr, live ? lane_u * 2u : kNoFetch, scale_plane + uni_u * 2u, 0);
    }
    // Unit metadata: z = 2^e (the unit's activation scale; the codes are
    // integers).
    __device__ static f32x4 meta(float /*gl*/, float /*gh*/, int e)
    {
        return f32x4{0.0f, 0.0f, __builtin_amdgcn_ldexpf(1.0f, e), 0.0f};
    }
    template <int N, int R, bool LO>
    __device__ static void accumulate(const Regs (&g)[R], const u32x4 *__restrict__ xs,
                                      int ul, int uc, uint32_t /*u*/,
                                      float (&acc)[R][N])
    {
#pragma unroll
        for (int t = 0; t < N; t++) {
            const u32x4 *xu = xs + xslot(t, ul, uc);
            const f32x4 mt = __builtin_bit_cast(f32x4, xu[8]);
            u32x4 xh[4], xl[4];
#pragma unroll
            for (int i = 0; i < 4; i++) {
                xh[i] = xu[2 * i];
                xl[i] = LO ? xu[2 * i + 1] : u32x4{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int r = 0; r < R; r++) {
                float a = 0.0f;
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const uint32_t lo = (i == 0 ? g[r].q0.x : i == 1 ? g[r].q0.y : i == 2 ? g[r].q0.z : g[r].q0.w) ^ 0x80808080u;
                    const uint32_t hi = (i == 0 ? g[r].q1.x : i == 1 ? g[r].q1.y : i == 2 ? g[r].q1.z : g[r].q1.w) ^ 0x80808080u;
                    const uint32_t p0 = q8_pair<0x64u, 0>(lo), p2 = q8_pair<0x64u, 1>(lo);
                    const uint32_t p1 = q8_pair<0x74u, 0>(hi), p3 = q8_pair<0x74u, 1>(hi);
                    a = dot2(p0, xh[i].x, a);
                    a = dot2(p1, xh[i].y, a);
                    a = dot2(p2, xh[i].z, a);
                    a = dot2(p3, xh[i].w, a);
                    if constexpr (LO) {
                        a = dot2(p0, xl[i].x, a);
                        a = dot2(p1, xl[i].y, a);
                        a = dot2(p2, xl[i].z, a);
                        a = dot2(p3, xl[i].w, a);
                    }
                }
                acc[r][t] = __builtin_fmaf(half_lo(g[r].d) * mt.z, a, acc[r][t]);
            }
        }
    }
};

// Q1_0: a unit is one block: a 32-bit code word (bit e = element e) and an
// fp16 scale d in the scale plane. The value is (2b - 1) d: each bit pair,
// moved to bits (0, 16) for L elements (b*2^-24 as fp16 subnormals) or
// (4, 20) for H elements (16b*2^-24; their staged activations are divided by
// 16), becomes the exact normal codes (2b - 1)*2^-14 (16(2b - 1)*2^-14) by
// one packed fp16 fma (times 2048, less 2^-14 (16*2^-14)), so dot2 forms the
// unit's sum of (2b - 1) x directly.
// Pair order as staged: (L, L+2), (H, H+2), (L+1, L+3), (H+1, H+3) with
// L = 4i, H = L + 16 for item i, i.e. bits 4i.. of the word shifted down.
struct FmtQ1_0 {
    static constexpr int kFormat = Q4_FMT_Q1_0;
    static constexpr int kHighOffset = 16;
    static constexpr int kBatchUnits = 8;  // 6 B per unit
    __device__ static int unit_base(int u) { return u << 5; }
    __device__ static int item_base(int u, int i) { return unit_base(u) + 4 * i; }
    __device__ static uint32_t scale_plane(uint64_t rows, uint64_t k) { return static_cast<uint32_t>(rows * k / 8u); }

    struct Regs {
        uint32_t q;
        uint32_t d;
    };
    // Unit (row, u), row = trow + rowrel, u = ubase + li + jl: its code word
    // at (row*nu + u)*4, its scale at scale_plane + (row*nu + u)*2.
    __device__ static void load(Regs &g, __amdgpu_buffer_rsrc_t wr, uint32_t scale_plane, uint32_t nu,
                                uint32_t trow, uint32_t rowrel, uint32_t li, uint32_t ubase, uint32_t jl, bool live)
    {
        const uint32_t uni_u = uniform(trow * nu + ubase);
        const uint32_t lane_u = rowrel * nu + li + jl;
        g.q = __builtin_amdgcn_raw_buffer_load_b32(wr, live ? lane_u * 4u : kNoFetch, uni_u * 4u, kNonTemporal);
        g.d = __builtin_amdgcn_raw_buffer_load_b16(wr, live ? lane_u * 2u : kNoFetch, scale_plane + uni_u * 2u, 0);
    }
    // Unit metadata: z = 2^(e+14) (the unit's activation scale times the
    // codes' factor 2^14).
    __device__ static f32x4 meta(float /*gl*/, float /*gh*/, int e)
    {
        return f32x4{0.0f, 0.0f, __builtin_amdgcn_ldexpf(1.0f, e + kCodeExp), 0.0f};
    }
    // Bits v*2^-24 (v = b or 16b per half) -> exact fp16 pair
    // (2v - OFF)*2^-14 = 2048 * v*2^-24 - OFF*2^-14.
    template <int OFF>
    __device__ static uint32_t sign_pair(uint32_t v)
    {
        const half2_t h = __builtin_bit_cast(half2_t, v);
        const _Float16 k = static_cast<_Float16>(2048.0f);
        const _Float16 o = static_cast<_Float16>(-static_cast<float>(OFF) * 0x1p-14f);
        return __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(h, half2_t{k, k}, half2_t{o, o}));
    }
    // Code pairs of item i from t = word >> 4i: L pairs take bits (0, 2) and
    // (1, 3) to bits (0, 16); H pairs take bits (16, 18) and (17, 19) to
    // bits (4, 20).
    __device__ static uint32_t pair_l0(uint32_t t) { return (t & 1u) | ((t << 14) & 0x10000u); }
    __device__ static uint32_t pair_h0(uint32_t t) { return ((t >> 12) & 0x10u) | ((t << 2) & 0x100000u); }
    __device__ static uint32_t pair_l1(uint32_t t) { return ((t >> 1) & 1u) | ((t << 13) & 0x10000u); }
    __device__ static uint32_t pair_h1(uint32_t t) { return ((t >> 13) & 0x10u) | ((t << 1) & 0x100000u); }
    template <int N, int R, bool LO>
    __device__ static void accumulate(const Regs (&g)[R], const u32x4 *__restrict__ xs,
                                      int ul, int uc, uint32_t /*u*/,
                                      float (&acc)[R][N])
    {
#pragma unroll
        for (int t = 0; t < N; t++) {
            const u32x4 *xu = xs + xslot(t, ul, uc);
            const f32x4 mt = __builtin_bit_cast(f32x4, xu[8]);
            u32x4 xh[4], xl[4];
#pragma unroll
            for (int i = 0; i < 4; i++) {
                xh[i] = xu[2 * i];
                xl[i] = LO ? xu[2 * i + 1] : u32x4{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int r = 0; r < R; r++) {
                float a = 0.0f;
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const uint32_t tt = g[r].q >> (4 * i);
                    const uint32_t p0 = sign_pair<1>(pair_l0(tt)), p1 = sign_pair<16>(pair_h0(tt));
                    const uint32_t p2 = sign_pair<1>(pair_l1(tt)), p3 = sign_pair<16>(pair_h1(tt));
                    a = dot2(p0, xh[i].x, a);
                    a = dot2(p1, xh[i].y, a);
                    a = dot2(p2, xh[i].z, a);
                    a = dot2(p3, xh[i].w, a);
                    if constexpr (LO) {
                        a = dot2(p0, xl[i].x, a);
                        a = dot2(p1, xl[i].y, a);
                        a = dot2(p2, xl[i].z, a);
                        a = dot2(p3, xl[i].w, a);
                    }
                }
                acc[r][t] = __builtin_fmaf(half_lo(g[r].d) * mt.z, a, acc[r][t]);
            }
        }
    }
};

// Q2_K: unit u = 8 code bytes of super-block u >> 3: bytes 32h + 8i .. +7
// of its 64 code bytes, h = (u & 7) >> 2, i = u & 3. Those bytes hold, in
// bit pairs 2j, 2j+1, the codes of the four runs j = 0..3 of 8 elements
// 128h + 32j + 8i .. +7; run j lies in sub-block 8h + 2j + (i >= 2). Item j
// of the unit is run j: L = its first four elements, H = its last four
// (kHighOffset 4, staged divided by 16). A code pair is the masked bits (an
// fp16 subnormal pair) times 1024: q*2^-14 (L) or 16q*2^-14 (H), exact
// normal fp16 values or zero.
template <int J>
__device__ __forceinline__ uint32_t q2_hi_pair(uint32_t b)
{
    // Bits 2J, 2J+1 of bytes 0 and 2 moved to bits 4, 5 of each half.
    if constexpr (J < 2) return (b << (4 - 2 * J)) & 0x00300030u;
    else return (b >> (2 * J - 4)) & 0x00300030u;
}

struct FmtQ2_K {
    static constexpr int kFormat = Q4_FMT_Q2_K;
    static constexpr int kHighOffset = 4;
    static constexpr int kBatchUnits = 4;  // 8 code bytes, 8 scale bytes and d, dmin per unit
    __device__ static int item_base(int u, int i) { return ((u >> 3) << 8) + (((u & 7) >> 2) << 7) + 32 * i + 8 * (u & 3); }
    // Offset of the scale plane; the d, dmin plane follows it at a quarter of its offset.
    __device__ static uint32_t scale_plane(uint64_t rows, uint64_t k) { return static_cast<uint32_t>(rows * k / 4u); }

    struct Regs {
        u32x2 q;   // 8 code bytes
        u32x2 sc;  // scale bytes 8h .. 8h+7 of the super-block
        uint32_t dd;  // fp16 d | fp16 dmin << 16
    };
    // Unit u = ubase + li + jl of row trow + rowrel (ubase and jl multiples of
    // 8): super-block (row*ns + u/8); code bytes at 64 per super-block + 8*(u & 7),
    // scale bytes at scale_plane + 16 per super-block + 8h, d and dmin at
    // scale_plane*5/4 + 4 per super-block.
    __device__ static void load(Regs &g, __amdgpu_buffer_rsrc_t wr, uint32_t scale_plane, uint32_t nu,
                                uint32_t trow, uint32_t rowrel, uint32_t li, uint32_t ubase, uint32_t jl, bool live)
    {
        const uint32_t ns = nu >> 3;
        const uint32_t uni_sb = uniform(trow * ns + (ubase >> 3));
        const uint32_t lane_sb = rowrel * ns + (li >> 3) + (jl >> 3);
        const uint32_t dd_plane = scale_plane + scale_plane / 4u;
        g.q = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(
                                            wr, live ? lane_sb * 64u + 8u * (li & 7u) : kNoFetch, uni_sb * 64u,
                                            kNonTemporal));
        g.sc = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(
                                             wr, live ? lane_sb * 16u + 8u * ((li & 7u) >> 2) : kNoFetch,
                                             scale_plane + uni_sb * 16u, 0));
        g.dd = __builtin_amdgcn_raw_buffer_load_b32(wr, live ? lane_sb * 4u : kNoFetch, dd_plane + uni_sb * 4u, 0);
    }
    // Unit metadata: z = 2^(e+14) (the codes carry 2^-14), w = 2^e.
    __device__ static f32x4 meta(float /*gl*/, float /*gh*/, int e)
    {
        return f32x4{0.0f, 0.0f, __builtin_amdgcn_ldexpf(1.0f, e + kCodeExp), __builtin_amdgcn_ldexpf(1.0f, e)};
    }
    template <int N, int R, bool LO>
    __device__ static void accumulate(const Regs (&g)[R], const u32x4 *__restrict__ xs,
                                      int ul, int uc, uint32_t u,
                                      float (&acc)[R][N])
    {
        constexpr uint32_t one = 0x3C003C00u, sixteen = 0x4C004C00u;  // fp16 pairs (1, 1) and (16, 16)
        const uint32_t c = (u & 3u) >> 1;  // runs of units i >= 2 lie in the odd sub-blocks
        float dsc[R][4], dmn[R][4];
#pragma unroll
        for (int r = 0; r < R; r++) {
            const float d = half_lo(g[r].dd), dmin = half_hi(g[r].dd);
#pragma unroll
            for (int j = 0; j < 4; j++) {
                // Scale byte 2j + c of the 8 loaded: dword j >> 1, byte 2(j & 1) + c.
                const uint32_t word = (j >> 1) ? g[r].sc.y : g[r].sc.x;
                const uint32_t byte = (word >> (8u * (2u * (j & 1) + c))) & 0xFFu;
                dsc[r][j] = d * static_cast<float>(byte & 15u);
                dmn[r][j] = dmin * static_cast<float>(byte >> 4);
            }
        }
#pragma unroll
        for (int t = 0; t < N; t++) {
            const u32x4 *xu = xs + xslot(t, ul, uc);
            const f32x4 mt = __builtin_bit_cast(f32x4, xu[8]);
            u32x4 xh[4], xl[4];
            float sx[4];
#pragma unroll
            for (int j = 0; j < 4; j++) {
                xh[j] = xu[2 * j];
                xl[j] = LO ? xu[2 * j + 1] : u32x4{0u, 0u, 0u, 0u};
                // Sum of the run's staged activations (the H ones counted 16 times).
                float s = dot2(xh[j].x, one, 0.0f);
                s = dot2(xh[j].y, sixteen, s);
                s = dot2(xh[j].z, one, s);
                s = dot2(xh[j].w, sixteen, s);
                if constexpr (LO) {
                    s = dot2(xl[j].x, one, s);
                    s = dot2(xl[j].y, sixteen, s);
                    s = dot2(xl[j].z, one, s);
                    s = dot2(xl[j].w, sixteen, s);
                }
                sx[j] = s;
            }
#pragma unroll
            for (int r = 0; r < R; r++) {
                const uint32_t a = g[r].q.x, b = g[r].q.y;
                float ts = 0.0f, tm = 0.0f;
                auto run = [&](auto jc) {
                    constexpr int j = decltype(jc)::value;
                    const uint32_t p0 = code_pair<0>((a >> (2 * j)) & 0x00030003u);
                    const uint32_t p2 = code_pair<0>((a >> (2 * j + 8)) & 0x00030003u);
                    const uint32_t p1 = code_pair<0>(q2_hi_pair<j>(b));
                    const uint32_t p3 = code_pair<0>((b >> (2 * j + 4)) & 0x00300030u);
                    float aj = dot2(p0, xh[j].x, 0.0f);
                    aj = dot2(p1, xh[j].y, aj);
                    aj = dot2(p2, xh[j].z, aj);
                    aj = dot2(p3, xh[j].w, aj);
                    if constexpr (LO) {
                        aj = dot2(p0, xl[j].x, aj);
                        aj = dot2(p1, xl[j].y, aj);
                        aj = dot2(p2, xl[j].z, aj);
                        aj = dot2(p3, xl[j].w, aj);
                    }
                    ts = __builtin_fmaf(dsc[r][j], aj, ts);
                    tm = __builtin_fmaf(dmn[r][j], sx[j], tm);
                };
                run(std::integral_constant<int, 0>{});
                run(std::integral_constant<int, 1>{});
                run(std::integral_constant<int, 2>{});
                run(std::integral_constant<int, 3>{});
                acc[r][t] = __builtin_fmaf(mt.z, ts, acc[r][t]);
                acc[r][t] = __builtin_fmaf(-mt.w, tm, acc[r][t]);
            }
        }
    }
};

struct FmtQ4_K {
    static constexpr int kFormat = Q4_FMT_Q4_K;
    static constexpr int kHighOffset = 32;
    static constexpr int kBatchUnits = 2;  // each unit is two 16-byte loads
    __device__ static uint32_t scale_plane(uint64_t, uint64_t) { return 0; }  // headers are in the super-blocks
    // unit u = slice (u & 7) of super-block u >> 3; slice h covers the 16
    // bytes at 16h of the 128 nibble bytes: chunk c = h >> 1, half h & 1.
    __device__ static int unit_base(int u) { return ((u >> 3) << 8) + (((u & 7) >> 1) << 6) + ((u & 1) << 4); }
    __device__ static int item_base(int u, int i) { return unit_base(u) + 4 * i; }

    struct Regs {
        u32x4 q;
        u32x4 h;
    };
    // Unit u = ubase + li + jl of row trow + rowrel (ubase and jl multiples
    // of 8): super-block (row*ns + u/8) at 144 bytes each, header at its
    // start, slice u & 7 = li & 7 at 16 + 16*(li & 7).
    __device__ static void load(Regs &g, __amdgpu_buffer_rsrc_t wr, uint32_t /*scale_plane*/, uint32_t nu,
                                uint32_t trow, uint32_t rowrel, uint32_t li, uint32_t ubase, uint32_t jl, bool live)
    {
        const uint32_t ns = nu >> 3;
        const uint32_t uni_b = uniform((trow * ns + (ubase >> 3)) * 144u);
        const uint32_t lane_b = live ? (rowrel * ns + (li >> 3) + (jl >> 3)) * 144u : kNoFetch;
        g.h = load16<0>(wr, lane_b, uni_b);
        g.q = load16<kNonTemporal>(wr, lane_b + 16u + ((li & 7u) << 4), uni_b);
    }
    // Unit metadata: x = sum of the 16 low-nibble activations, y = 16 x sum of
    // the 16 pre-divided high-nibble activations (both scaled units),
    // z = 2^(e+14) (the codes carry 2^-14), w = 2^e.
    __device__ static f32x4 meta(float gl, float gh, int e)
    {
        return f32x4{gl, gh, __builtin_amdgcn_ldexpf(1.0f, e + kCodeExp), __builtin_amdgcn_ldexpf(1.0f, e)};
    }
    template <int N, int R, bool LO>
    __device__ static void accumulate(const Regs (&g)[R], const u32x4 *__restrict__ xs,
                                      int ul, int uc, uint32_t u,
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
            const u32x4 *xu = xs + xslot(t, ul, uc);
            const f32x4 mt = __builtin_bit_cast(f32x4, xu[8]);
            u32x4 xh[4], xl[4];
#pragma unroll
            for (int i = 0; i < 4; i++) {
                xh[i] = xu[2 * i];
                xl[i] = LO ? xu[2 * i + 1] : u32x4{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int r = 0; r < R; r++) {
                float aa = 0.0f, ab = 0.0f;
                const u32x4 q = g[r].q;
                // Each dword: pairs 0 and 2 belong to sub-block a, 1 and 3 to b.
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const uint32_t qi = i == 0 ? q.x : i == 1 ? q.y : i == 2 ? q.z : q.w;
                    const uint32_t s = qi >> 8;
                    const uint32_t p0 = code_pair<0>(qi & kLo), p1 = code_pair<0>(qi & kHi);
                    const uint32_t p2 = code_pair<0>(s & kLo), p3 = code_pair<0>(s & kHi);
                    aa = dot2(p0, xh[i].x, aa);
                    ab = dot2(p1, xh[i].y, ab);
                    aa = dot2(p2, xh[i].z, aa);
                    ab = dot2(p3, xh[i].w, ab);
                    if constexpr (LO) {
                        aa = dot2(p0, xl[i].x, aa);
                        ab = dot2(p1, xl[i].y, ab);
                        aa = dot2(p2, xl[i].z, aa);
                        ab = dot2(p3, xl[i].w, ab);
                    }
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
// Units [c0, c0 + nuc) of every token -> LDS: planes (t, 2i) and (t, 2i+1)
// hold the hi and lo fp16 pairs for nibble dword i. Item (t, ul, i) handles dword i
// of unit ul: activations L..L+3 (low nibbles) and H..H+3 (high nibbles),
// L = item_base(unit, i) (unit_base + 4i for the nibble formats), H = L +
// kHighOffset. The four items of a unit are four
// consecutive lanes, which exchange their maxima and partial sums.

// The four items of a unit are one lane quad (every count and stride here is
// a multiple of 4), so their exchanges are DPP quad permutations.
template <int CTRL>
__device__ __forceinline__ float dpp(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

// Buffers of the fused residual add + RMSNorm (one token): the staged
// activation is (x + delta) * gain; `out` receives x + delta (its range is
// empty except in the one workgroup that writes it); ssq accumulates this
// thread's squares of x + delta.
struct NormIo {
    __amdgpu_buffer_rsrc_t delta, gain, out;
    float ssq;
};

// Round one of the staging issues P items' activation loads per thread, then
// calls issue() (the first weight batch), and only then waits for the
// activations, so the weight loads are in flight during the staging and the
// staging waits on one L2 round trip per round, not one per item.
template <class F, int N, int NT, int P, bool LO, bool NORM, class Issue, bool SKIP_DEAD = false>
__device__ __forceinline__ void stage(__amdgpu_buffer_rsrc_t xr, int K, int c0, int nuc, int uc,
                                      u32x4 *__restrict__ xs, int tid, NormIo &nio, Issue issue)
{
    static_assert(!NORM || N == 1, "the fused norm is a one-token prologue");
    const int per_tok = nuc * 4;
    const int total = N * per_tok;
    // it / per_tok as a multiply-high by ceil(2^32 / per_tok): exact while
    // it * per_tok < 2^32 (it < N * per_tok and per_tok <= 4 * 163840 / (144 N)
    // here, the most units one workgroup's LDS holds for N >= 2 tokens).
    const uint32_t inv = N == 1 ? 0u : 0xFFFFFFFFu / static_cast<uint32_t>(per_tok) + 1u;
    auto split_item = [&](int it, int &t, int &rem) {
        if constexpr (N == 1) {
            t = 0;
            rem = it;
        } else {
            t = static_cast<int>(__umulhi(static_cast<uint32_t>(it), inv));
            rem = it - t * per_tok;
        }
    };
    bool issued = false;
    for (int rb = 0; rb < total || !issued; rb += P * NT) {
        const int base = rb + tid;
        f32x4 a[P], b[P], da[P], db[P], ga[P], gb[P];
        uint32_t offs[P];
#pragma unroll
        for (int p = 0; p < P; p++) {
            // Lanes past the end land past N*K and read zeros. With SKIP_DEAD
            // a slot with no live item in the whole workgroup issues no loads
            // at all (a uniform branch: even a load that fetches nothing costs
            // the CU's address unit a pass over 64 lanes); without it every
            // slot's loads are issued, branch-free.
            const f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
            a[p] = b[p] = da[p] = db[p] = ga[p] = gb[p] = z;
            offs[p] = 0u;
            if (SKIP_DEAD && rb + p * NT >= total) continue;
            int t, rem;
            split_item(base + p * NT, t, rem);
            const uint32_t off = static_cast<uint32_t>(t * K + F::item_base(c0 + (rem >> 2), rem & 3)) * 4u;
            offs[p] = off;
            a[p] = __builtin_bit_cast(f32x4, load16<0>(xr, off, 0));
            b[p] = __builtin_bit_cast(f32x4, load16<0>(xr, off + 4u * F::kHighOffset, 0));
            if constexpr (NORM) {
                da[p] = __builtin_bit_cast(f32x4, load16<0>(nio.delta, off, 0));
                db[p] = __builtin_bit_cast(f32x4, load16<0>(nio.delta, off + 4u * F::kHighOffset, 0));
                ga[p] = __builtin_bit_cast(f32x4, load16<0>(nio.gain, off, 0));
                gb[p] = __builtin_bit_cast(f32x4, load16<0>(nio.gain, off + 4u * F::kHighOffset, 0));
            }
        }
        if (!issued) {
            // Keep the scheduler from moving activation loads behind the weights.
            __builtin_amdgcn_sched_barrier(0);
            issue();
            issued = true;
        }
        // Every load above is consumed here, so none of them can be sunk into
        // the branches below (behind the weight loads, whose wait would then
        // cover them too).
#pragma unroll
        for (int p = 0; p < P; p++) asm volatile("" ::"v"(a[p]), "v"(b[p]));
        if constexpr (NORM) {
#pragma unroll
            for (int p = 0; p < P; p++) asm volatile("" ::"v"(da[p]), "v"(db[p]), "v"(ga[p]), "v"(gb[p]));
        }
#pragma unroll
        for (int p = 0; p < P; p++) {
            // Slots with no live item in the whole workgroup are skipped (a
            // uniform branch); in the last live slot, lanes past the end
            // compute on zeros and store nothing.
            if (rb + p * NT >= total) break;
            const bool live = base + p * NT < total;
            if constexpr (NORM) {
                // Residual add, its squares, its write-back (dead lanes hold
                // zeros at offsets past the end: nothing added or stored),
                // then the gain; the row's 1/rms scales the reduced sums.
                a[p] += da[p];
                b[p] += db[p];
                float q = a[p].x * a[p].x;
                q = __builtin_fmaf(a[p].y, a[p].y, q);
                q = __builtin_fmaf(a[p].z, a[p].z, q);
                q = __builtin_fmaf(a[p].w, a[p].w, q);
                q = __builtin_fmaf(b[p].x, b[p].x, q);
                q = __builtin_fmaf(b[p].y, b[p].y, q);
                q = __builtin_fmaf(b[p].z, b[p].z, q);
                q = __builtin_fmaf(b[p].w, b[p].w, q);
                nio.ssq += q;
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, a[p]), nio.out, offs[p], 0, 0);
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, b[p]), nio.out,
                                                       offs[p] + 4u * F::kHighOffset, 0, 0);
                a[p] *= ga[p];
                b[p] *= gb[p];
            }
            int t, rem;
            split_item(live ? base + p * NT : 0, t, rem);
            const int ul = rem >> 2;
            const int i = rem & 3;
            float mx = __builtin_fmaxf(__builtin_fmaxf(__builtin_fabsf(a[p].x), __builtin_fabsf(a[p].y)),
                                       __builtin_fmaxf(__builtin_fabsf(a[p].z), __builtin_fabsf(a[p].w)));
            mx = __builtin_fmaxf(mx, __builtin_fmaxf(__builtin_fmaxf(__builtin_fabsf(b[p].x), __builtin_fabsf(b[p].y)),
                                                     __builtin_fmaxf(__builtin_fabsf(b[p].z), __builtin_fabsf(b[p].w))));
            mx = __builtin_fmaxf(mx, dpp<0xB1>(mx));  // quad_perm [1,0,3,2]
            mx = __builtin_fmaxf(mx, dpp<0x4E>(mx));  // quad_perm [2,3,0,1]
            // Largest magnitude -> [2^14, 2^15): x_tilde = x * 2^-e.
            const int e = __builtin_amdgcn_frexp_expf(mx) - 15;
            // Scaled activations (exact: power-of-two scaling); the high-nibble
            // ones pre-divided by 16 to cancel the 16x of their unpacked codes.
            const float l0 = __builtin_amdgcn_ldexpf(a[p].x, -e), l1 = __builtin_amdgcn_ldexpf(a[p].y, -e);
            const float l2 = __builtin_amdgcn_ldexpf(a[p].z, -e), l3 = __builtin_amdgcn_ldexpf(a[p].w, -e);
            const float h0 = __builtin_amdgcn_ldexpf(b[p].x, -e - 4), h1 = __builtin_amdgcn_ldexpf(b[p].y, -e - 4);
            const float h2 = __builtin_amdgcn_ldexpf(b[p].z, -e - 4), h3 = __builtin_amdgcn_ldexpf(b[p].w, -e - 4);
            const Split sl0 = split(l0), sl1 = split(l1), sl2 = split(l2), sl3 = split(l3);
            const Split sh0 = split(h0), sh1 = split(h1), sh2 = split(h2), sh3 = split(h3);
            const u32x4 vhi = u32x4{pack_h2(sl0.hi, sl2.hi), pack_h2(sh0.hi, sh2.hi), pack_h2(sl1.hi, sl3.hi),
                                    pack_h2(sh1.hi, sh3.hi)};
            const u32x4 vlo = u32x4{pack_h2(sl0.lo, sl2.lo), pack_h2(sh0.lo, sh2.lo), pack_h2(sl1.lo, sl3.lo),
                                    pack_h2(sh1.lo, sh3.lo)};
            float gl = (l0 + l1) + (l2 + l3);
            float gh = (h0 + h1) + (h2 + h3);
            gl += dpp<0xB1>(gl);
            gh += dpp<0xB1>(gh);
            gl += dpp<0x4E>(gl);
            gh += dpp<0x4E>(gh);
            const f32x4 mv = F::meta(gl, 16.0f * gh, e);
            if (live) {
                u32x4 *dst = xs + xslot(t, ul, uc);
                dst[2 * i] = vhi;
                if constexpr (LO) dst[2 * i + 1] = vlo;
                if (i == 0) dst[8] = __builtin_bit_cast(u32x4, mv);
            }
        }
    }
}

// ---- cross-lane row reduction ------------------------------------------------------
// Sum over the LPR consecutive lanes of a sub-group; the total lands in the
// sub-group's first lane. Quad and row steps use DPP (quad_perm, row_ror);
// steps across 16-lane rows use a lane shuffle.

template <int CTRL>
__device__ __forceinline__ float dpp_add(float v)
{
    return v + dpp<CTRL>(v);
}

template <int LPR>
__device__ __forceinline__ float row_reduce(float v)
{
    v = dpp_add<0xB1>(v);               // quad_perm [1,0,3,2]: + lane ^ 1
    v = dpp_add<0x4E>(v);               // quad_perm [2,3,0,1]: + lane ^ 2
    // row_ror:N moves data N lanes up within a 16-lane row (lane i reads lane
    // i-N mod 16), so row_ror:12 makes lane i read lane i+4.
    if constexpr (LPR >= 8) v = dpp_add<0x12C>(v);   // row_ror:12: + lane (i+4) mod 16
    if constexpr (LPR >= 16) v = dpp_add<0x128>(v);  // row_ror:8: + lane (i+8) mod 16
    if constexpr (LPR >= 32) v += __shfl_down(v, 16);
    if constexpr (LPR >= 64) v += __shfl_down(v, 32);
    return v;
}

// ---- gated epilogue ------------------------------------------------------------------
// The gate and up projections of a gated MLP share their input, so one launch
// computes both and applies the activation to the gate: silu(g) * u, with
// silu(g) = g / (1 + e^-g) (kernel fusion: WebGPT README, "Roadmap"; the
// technical summary of Llamas on the Web credits fused kernels for prefill
// throughput in its experimental results).
__device__ __forceinline__ float silu_mul(float g, float u)
{
    return g / (1.0f + expf(-g)) * u;
}

// ---- the kernel -------------------------------------------------------------------
// Workgroup = WAVES waves; a tile is RPG = WAVES * (64/LPR) * R consecutive
// rows. In a tile, wave v covers rows v*RPW .. v*RPW + RPW - 1 (RPW =
// (64/LPR)*R): sub-group s (lanes s*LPR .. s*LPR+LPR-1) handles rows
// s + r*(64/LPR), r < R. Lane li of a sub-group handles units li, li+LPR, ...
// of each of its rows, JB unit slots per batch. Workgroups stride over the
// tiles (grid = min(tiles, resident capacity)), so the activations are staged
// once per workgroup when they fit in LDS; weight batches are double-buffered
// across tile boundaries, with the first batch issued before the staging.
// When the activations do not fit (many tokens x long rows) the row is
// processed in LDS-sized chunks, restaged per tile.
//
// GLU (R even): the weight matrix has 2M rows, gate rows 0..M-1 then up rows
// M..2M-1, and the output has M rows. A tile is then RPG/2 output rows; the
// lane's row slots pair up, slot 2p holding gate row o and slot 2p+1 up row
// M + o of the same output o = tile*RPG/2 + wave*RPW/2 + sub + p*(64/LPR).
// Each row's sum is formed exactly as in the plain product (same lanes, same
// order), and the epilogue applies silu_mul to the two reduced sums.
//
// NORM (one token, whole row staged): the input is rmsnorm(x + delta) *
// gain. Staging forms v = x + delta, stages v * gain and sums v^2; workgroup
// 0 also writes v to pro.x_out. As W (r v * gain) = r W (v * gain), the
// factor r = 1/sqrt(mean(v^2) + eps) multiplies each reduced row sum (before
// the gated epilogue). Every workgroup forms the same sum of squares (the
// same items, lanes and order), so every row sees the same r.

template <class F, int N, int LPR, int R, int WAVES, int JB, bool LO, bool GLU = false, bool NORM = false>
__global__ __launch_bounds__(64 * WAVES) void gemv_kernel(const uint8_t *__restrict__ w, uint32_t wbytes,
                                                          const float *__restrict__ x,
                                                          float *__restrict__ y, int M, int K, int uc,
                                                          int ntiles, Prologue pro)
{
    static_assert(!GLU || R % 2 == 0, "the gated product pairs row slots");
    static_assert(!NORM || N == 1, "the fused norm is a one-token prologue");
    constexpr int SUBS = 64 / LPR;
    constexpr int RPW = SUBS * R;
    constexpr int RPG = WAVES * RPW;
    constexpr int OPG = GLU ? RPG / 2 : RPG;  // output rows per tile
    constexpr int RO = GLU ? R / 2 : R;       // output rows per lane
    constexpr int NT = 64 * WAVES;
    extern __shared__ u32x4 lds[];
    u32x4 *xs = lds;
    float *wave_ssq = reinterpret_cast<float *>(lds + N * kLdsSlots * uc);  // NORM: one sum per wave

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int sub = lane / LPR;
    const int li = lane % LPR;
    const int nu = K >> 5;
    const uint64_t wrows = GLU ? 2ull * static_cast<uint64_t>(M) : static_cast<uint64_t>(M);
    const uint32_t scale_plane = F::scale_plane(wrows, static_cast<uint64_t>(K));
    // Output row of slot r (an output slot for the stores, a weight-row slot
    // for the loads: for GLU, slots 2p and 2p+1 share output slot p).
    const int out_in_tile = wave * (RPW / (GLU ? 2 : 1)) + sub;
    auto out_row = [&](int tile, int ro) { return tile * OPG + out_in_tile + ro * SUBS; };
    // Weight row of load slot r relative to the tile's first output row.
    auto wrow_rel = [&](int r) {
        return GLU ? out_in_tile + (r >> 1) * SUBS + (r & 1) * M : out_in_tile + r * SUBS;
    };
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, static_cast<uint32_t>(N) * static_cast<uint32_t>(K) * 4u);
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(w, wbytes);

    float acc[R][N];
    auto zero_acc = [&]() {
#pragma unroll
        for (int r = 0; r < R; r++)
#pragma unroll
            for (int t = 0; t < N; t++) acc[r][t] = 0.0f;
    };
    zero_acc();

    using Regs = typename F::Regs;

    // Batch of JB unit slots (units c0 + li + (j0+jj)*LPR) of the lane's R rows
    // in tile `tile`. Branch-free buffer loads that never fault: a slot past the
    // end of the chunk and a row past M (also every row of a tile past the
    // last) load from kNoFetch and read as zero without touching memory; such
    // slots are skipped in compute_batch and such rows are never stored. With
    // no branch around them the compiler counts every load as issued, so
    // waiting for one batch never waits for the next.
    auto load_batch = [&](Regs(&g)[JB][R], int tile, int j0, int c0, int nuc) {
        const uint32_t trow = static_cast<uint32_t>(tile) * OPG;
        const uint32_t ubase = static_cast<uint32_t>(c0 + j0 * LPR);
#pragma unroll
        for (int jj = 0; jj < JB; jj++)
#pragma unroll
            for (int r = 0; r < R; r++) {
                const bool live = li + (j0 + jj) * LPR < nuc && out_row(tile, GLU ? r >> 1 : r) < M;
                F::load(g[jj][r], wr, scale_plane, static_cast<uint32_t>(nu), trow,
                        static_cast<uint32_t>(wrow_rel(r)), static_cast<uint32_t>(li), ubase,
                        static_cast<uint32_t>(jj * LPR), live);
            }
    };
    auto compute_batch = [&](const Regs(&g)[JB][R], int j0, int c0, int nuc) {
#pragma unroll
        for (int jj = 0; jj < JB; jj++) {
            const int ul = li + (j0 + jj) * LPR;
            if (ul < nuc) F::template accumulate<N, R, LO>(g[jj], xs, ul, uc, static_cast<uint32_t>(c0 + ul), acc);
        }
    };
    // 1/rms of the fused norm (set once the staging is complete).
    float rn = 1.0f;
    auto scaled = [&](float v) {
        if constexpr (NORM)
            return v * rn;
        else
            return v;
    };
    // Reduced output value of output slot ro, token t.
    auto finish = [&](int ro, int t) {
        if constexpr (GLU)
            return silu_mul(scaled(row_reduce<LPR>(acc[2 * ro][t])), scaled(row_reduce<LPR>(acc[2 * ro + 1][t])));
        else
            return scaled(row_reduce<LPR>(acc[ro][t]));
    };
    auto reduce_store = [&](int tile) {
#pragma unroll
        for (int ro = 0; ro < RO; ro++) {
            const int row = out_row(tile, ro);
#pragma unroll
            for (int t = 0; t < N; t++) {
                const float v = finish(ro, t);
                if (li == 0 && row < M) y[static_cast<size_t>(t) * M + row] = v;
            }
        }
    };
    // The same stores issued in every step of the batch stream, writing only
    // at the end of a tile (elsewhere the offset is out of range and the
    // store is dropped): stores count in the same wait counter as loads, so
    // a store on only some paths makes the compiler's wait at the top of the
    // loop cover every outstanding load. Only the reduction, which touches
    // no memory, sits behind the (uniform) branch.
    const __amdgpu_buffer_rsrc_t yr = make_rsrc(y, static_cast<uint32_t>(N) * static_cast<uint32_t>(M) * 4u);
    auto store_if_end = [&](int tile, bool end) {
#pragma unroll
        for (int ro = 0; ro < RO; ro++) {
            const int row = out_row(tile, ro);
#pragma unroll
            for (int t = 0; t < N; t++) {
                float v = 0.0f;
                if (end) v = finish(ro, t);
                const bool live = end && li == 0 && row < M;
                __builtin_amdgcn_raw_buffer_store_b32(
                    __builtin_bit_cast(uint32_t, v), yr,
                    live ? (static_cast<uint32_t>(t) * static_cast<uint32_t>(M) + static_cast<uint32_t>(row)) * 4u
                         : kNoFetch,
                    0, 0);
            }
        }
    };

    int tile = blockIdx.x;
    if (tile >= ntiles) return;  // uniform across the workgroup
    Regs ga[JB][R], gb[JB][R];
    NormIo nio{xr, xr, xr, 0.0f};
    if constexpr (NORM) {
        const uint32_t kb = static_cast<uint32_t>(K) * 4u;
        nio.delta = make_rsrc(pro.delta, pro.delta ? kb : 0u);
        nio.gain = make_rsrc(pro.gain, kb);
        nio.out = make_rsrc(pro.x_out, pro.x_out && blockIdx.x == 0 ? kb : 0u);
    }

    if (uc >= nu) {
        // Activations staged once; a flat stream of batches runs through all
        // of this workgroup's tiles. Stream position = (tile, batch). Loads
        // run D batches ahead of the compute (D + 1 register buffers, used in
        // rotation), the first D issued before the staging waits. Every phase
        // issues the same loads and stores, so the compiler's wait counts stay
        // exact; the exit is a uniform branch between phases. (At one token the
        // batches are VALU-bound once staged: deeper prefetch, tried up to three
        // batches, only delays the activation loads behind weight traffic.)
        constexpr int D = 1;
        constexpr int NBUF = D + 1;
        const int nb = ((nu + LPR - 1) / LPR + JB - 1) / JB;  // batches per tile
        const int gstride = static_cast<int>(gridDim.x);
        int lt = tile, lb = 0;  // next position to load (past the last tile: no fetch)
        int ct = tile, cb = 0;  // next position to compute
        Regs gbuf[NBUF][JB][R];
        auto load_next = [&](Regs(&g)[JB][R]) {
            load_batch(g, lt, lb * JB, 0, nu);
            if (++lb == nb) {
                lb = 0;
                lt += gstride;
            }
        };
        auto compute_next = [&](const Regs(&g)[JB][R]) {
            compute_batch(g, cb * JB, 0, nu);
            const bool end = ++cb == nb;
            store_if_end(ct, end);
            if (end) {
                zero_acc();
                cb = 0;
                ct += gstride;
            }
        };
        stage<F, N, NT, kStageRound<WAVES>, LO, NORM>(xr, K, 0, nu, uc, xs, tid, nio, [&]() {
#pragma unroll
            for (int p = 0; p < D; p++) load_next(gbuf[p]);
        });
        if constexpr (NORM) {
            const float s = row_reduce<64>(nio.ssq);
            if (lane == 0) wave_ssq[wave] = s;
        }
        wg_sync<WAVES>();
        if constexpr (NORM) {
            float s = 0.0f;
#pragma unroll
            for (int v = 0; v < WAVES; v++) s += wave_ssq[v];
            rn = 1.0f / __builtin_sqrtf(s / static_cast<float>(K) + pro.eps);
        }
        for (;;) {
#pragma unroll
            for (int p = 0; p < NBUF; p++) {
                load_next(gbuf[(p + D) % NBUF]);
                compute_next(gbuf[p]);
                if (ct >= ntiles) goto stream_done;
            }
        }
    stream_done:
        return;
    }

    if constexpr (NORM) return;  // the host stages the whole row for the fused norm
    bool first = true;
    for (; tile < ntiles; tile += static_cast<int>(gridDim.x)) {
        for (int c0 = 0; c0 < nu; c0 += uc) {
            const int nuc = nu - c0 < uc ? nu - c0 : uc;
            const int jc = (nuc + LPR - 1) / LPR;  // unit slots per lane per row in this chunk
            if (!first) wg_sync<WAVES>();
            first = false;
            stage<F, N, NT, kStageRound<WAVES>, LO, false>(xr, K, c0, nuc, uc, xs, tid, nio,
                                                       [&]() { load_batch(ga, tile, 0, c0, nuc); });
            wg_sync<WAVES>();
            // Prefetches are unconditional (a batch past the chunk issues
            // no-fetch loads and is dropped) so that no branch makes the
            // compiler wait for them.
            for (int j0 = 0; j0 < jc; j0 += 2 * JB) {
                load_batch(gb, tile, j0 + JB, c0, nuc);
                compute_batch(ga, j0, c0, nuc);
                if (j0 + JB >= jc) break;
                load_batch(ga, tile, j0 + 2 * JB, c0, nuc);
                compute_batch(gb, j0 + JB, c0, nuc);
            }
        }
        reduce_store(tile);
        zero_acc();
    }
}

// ---- launch -----------------------------------------------------------------------

// m is the number of output rows (for GLU the weights have 2m rows).
template <class F, int N, int LPR, int R, int WAVES, bool GLU = false, bool NORM = false>
int launch_one(const uint8_t *w, const float *x, float *y, int m, int k, hipStream_t stream, int cus,
               int groups_per_cu, const Prologue &pro = Prologue{})
{
    constexpr int JB = F::kBatchUnits / R > 0 ? F::kBatchUnits / R : 1;
    constexpr int rows_per_wg = WAVES * (64 / LPR) * R / (GLU ? 2 : 1);
    const int nu = k / 32;
    int uc = nu;
    const int bytes_per_unit = N * kLdsBytesPerUnit;
    // Several tokens of a long row exceed the default 64 KiB: rather than
    // restage the activations chunk by chunk for every tile, take up to the
    // workgroup's opt-in LDS (160 KiB on gfx950), which holds the whole row
    // (8 tokens of 4096, 4 of 8960) or larger chunks, at fewer groups per CU.
    // (64-bit products: a whole row of many tokens can exceed 2^31 bytes.)
    const int64_t row_bytes = static_cast<int64_t>(nu) * bytes_per_unit;
    const int extra = NORM ? 4 * WAVES : 0;  // the fused norm's per-wave sums of squares
    int budget = kMaxLdsBytes;
    if ((NORM || N >= 2) && row_bytes + extra > kMaxLdsBytes) {
        const int optin = device_lds_optin();
        if (optin > kMaxLdsBytes) budget = optin;
    }
    if (row_bytes + extra > budget) uc = (budget - extra) / bytes_per_unit / 8 * 8;  // chunks of whole super-blocks
    if (uc <= 0) return Q4_EUNSUPPORTED;
    if (NORM && uc < nu) return Q4_EUNSUPPORTED;  // the fused norm needs the whole row staged
    const size_t lds = static_cast<size_t>(uc) * bytes_per_unit + extra;
    if (lds > static_cast<size_t>(kMaxLdsBytes)) {
        // Above 64 KiB a kernel opts in to its dynamic LDS size, once per device.
        static std::atomic<int> opted[64];
        int dev = 0;
        if (hip_status(hipGetDevice(&dev)) != Q4_OK) return Q4_EHIP;
        if (dev < 0 || dev >= 64) return Q4_EUNSUPPORTED;
        if (!opted[dev].load(std::memory_order_acquire)) {
            int st = hip_status(hipFuncSetAttribute(
                reinterpret_cast<const void *>(&gemv_kernel<F, N, LPR, R, WAVES, JB, true, GLU, NORM>),
                hipFuncAttributeMaxDynamicSharedMemorySize, budget));
            if (st == Q4_OK)
                st = hip_status(hipFuncSetAttribute(
                    reinterpret_cast<const void *>(&gemv_kernel<F, N, LPR, R, WAVES, JB, false, GLU, NORM>),
                    hipFuncAttributeMaxDynamicSharedMemorySize, budget));
            if (st != Q4_OK) return st;
            opted[dev].store(1, std::memory_order_release);
        }
        // Groups that fit a compute unit's LDS at once.
        const int fit = budget / static_cast<int>(lds);
        if (groups_per_cu > fit) groups_per_cu = fit > 0 ? fit : 1;
    }
    const int ntiles = (m + rows_per_wg - 1) / rows_per_wg;
    const long long cap = static_cast<long long>(cus) * groups_per_cu;
    const unsigned grid = static_cast<unsigned>(ntiles < cap ? ntiles : cap);
    const int64_t wrows = GLU ? 2 * static_cast<int64_t>(m) : m;
    const uint32_t wbytes = static_cast<uint32_t>(q4_weight_bytes(F::kFormat, wrows, k));
    // Activations as hi + lo fp16 pairs (about 2^-23 relative) for short
    // matrices, as one fp16 each (2^-11 relative, half the dot issues, LDS
    // reads and staging work) once there are kLoRowLimit rows or more
    // (weight rows: a gated product rounds like the plain product of its
    // stacked matrix).
    if (wrows < kLoRowLimit)
        hipLaunchKernelGGL((gemv_kernel<F, N, LPR, R, WAVES, JB, true, GLU, NORM>), dim3(grid), dim3(64 * WAVES), lds,
                           stream, w, wbytes, x, y, m, k, uc, ntiles, pro);
    else
        hipLaunchKernelGGL((gemv_kernel<F, N, LPR, R, WAVES, JB, false, GLU, NORM>), dim3(grid), dim3(64 * WAVES), lds,
                           stream, w, wbytes, x, y, m, k, uc, ntiles, pro);
    return hip_status(hipGetLastError());
}

// The instantiated tile geometries: (lanes per row, rows per lane, waves per group).
#define Q4_GEMV_CONFIGS(X) \
    X(8, 1, 1)             \
    X(8, 2, 1)             \
    X(8, 4, 1)             \
    X(16, 1, 1)            \
    X(16, 2, 1)            \
    X(32, 1, 1)            \
    X(32, 2, 1)            \
    X(64, 1, 1)            \
    X(16, 1, 4)            \
    X(32, 1, 4)            \
    X(32, 2, 4)            \
    X(64, 1, 4)            \
    X(64, 2, 4)            \
    X(64, 4, 4)            \
    X(32, 1, 8)

template <class F, int N>
int dispatch_cfg(const Cfg &c, const uint8_t *w, const float *x, float *y, int m, int k, hipStream_t s, int cus)
{
#define Q4_CFG_CASE(L, RR, WV) \
    if (c.lpr == L && c.r == RR && c.waves == WV) return launch_one<F, N, L, RR, WV>(w, x, y, m, k, s, cus, c.groups_per_cu);
    Q4_GEMV_CONFIGS(Q4_CFG_CASE)
#undef Q4_CFG_CASE
    return Q4_EUNSUPPORTED;
}

// The gated product's geometries (two row slots per lane: a gate and an up row).
#define Q4_GEMV_GLU_CONFIGS(X) \
    X(16, 2, 1)                \
    X(16, 2, 4)                \
    X(32, 2, 1)                \
    X(32, 2, 4)                \
    X(32, 2, 8)                \
    X(64, 2, 4)

template <class F, int N>
int dispatch_glu_cfg(const Cfg &c, const uint8_t *w, const float *x, float *y, int m, int k, hipStream_t s, int cus)
{
#define Q4_CFG_CASE(L, RR, WV)                                   \
    if (c.lpr == L && c.r == RR && c.waves == WV)                \
        return launch_one<F, N, L, RR, WV, true>(w, x, y, m, k, s, cus, c.groups_per_cu);
    Q4_GEMV_GLU_CONFIGS(Q4_CFG_CASE)
#undef Q4_CFG_CASE
    return Q4_EUNSUPPORTED;
}

// The fused-norm product's geometries: every one-token choice of choose()
// and choose_glu().
#define Q4_GEMV_NORM_CONFIGS(X) \
    X(8, 1, 1)                  \
    X(8, 2, 1)                  \
    X(16, 1, 1)                 \
    X(16, 1, 4)                 \
    X(32, 1, 4)                 \
    X(32, 1, 8)                 \
    X(32, 2, 1)                 \
    X(32, 2, 4)                 \
    X(64, 1, 4)

template <class F>
int dispatch_norm_cfg(const Cfg &c, const uint8_t *w, const float *x, float *y, int m, int k, hipStream_t s, int cus,
                      bool glu, const Prologue &pro)
{
    static_assert(kMaxLdsBytes / kLdsBytesPerUnit == kNormMaxUnits, "fused-norm row limit");
#define Q4_CFG_CASE(L, RR, WV) \
    if (!glu && c.lpr == L && c.r == RR && c.waves == WV) \
        return launch_one<F, 1, L, RR, WV, false, true>(w, x, y, m, k, s, cus, c.groups_per_cu, pro);
    Q4_GEMV_NORM_CONFIGS(Q4_CFG_CASE)
#undef Q4_CFG_CASE
#define Q4_CFG_CASE(L, RR, WV) \
    if (glu && c.lpr == L && c.r == RR && c.waves == WV) \
        return launch_one<F, 1, L, RR, WV, true, true>(w, x, y, m, k, s, cus, c.groups_per_cu, pro);
    Q4_GEMV_GLU_CONFIGS(Q4_CFG_CASE)
#undef Q4_CFG_CASE
    return Q4_EUNSUPPORTED;
}

}  // namespace gemv
}  // namespace q4
