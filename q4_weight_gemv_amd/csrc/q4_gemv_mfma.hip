// Decode product at several tokens for Q4_K on gfx950's matrix cores.
//
// At 2 to 8 tokens the tiled kernel's VALU dot products bound it: every
// weight pair costs one v_dot2 per token. Here v_mfma_f32_16x16x32_f16 forms
// the products, so a weight costs its unpacking once, whatever the token
// count, and the weight stream is the bound again.
//
// Format (llama.cpp K-quants, the stretch format of Llamas on the Web,
// technical summary, Methodology section 3): a 256-weight super-block holds
// fp16 d and dmin, twelve bytes of 6-bit sub-block scales sc and mins m, and
// 128 nibble bytes; weight = d * sc * q - dmin * m for its 32-weight sub-block.
//
// Per super-block and tile of 16 weight rows, with tokens on the MFMA's A side
// (16 slots; the unused ones repeat token 0 and are never stored) and weight
// rows on its B side:
//   Dq[t][r] = sum_k (sc q)[r][k] * xs[t][k]      eight MFMAs
//   Dm[t][r] = sum_k m[r][s(k)] * xs[t][k]         eight MFMAs (the sub-block's min, broadcast)
//   y[t][r] += 2^e[t] * (d[r] Dq[t][r] - dmin[r] Dm[t][r])
// where xs = x * 2^-e[t] rounded to fp16, e[t] per token and super-block
// putting its largest magnitude into [2^14, 2^15). sc q (at most 945) and m
// (at most 63) are exact fp16 values and every product is exact in fp32, so
// the only roundings are x's to fp16 (at most 2^-11 relative) and the fp32 sums.
//
// MFMA 16x16x32 operand layout (wave64): lane l holds A row l%16 (a token)
// and B column l%16 (a weight row), each at the 8 k slots 8(l/16)..+7; the
// result D[4(l/16)+i][l%16], i < 4. Within a super-block, MFMA j (0..7) gives
// lane group g = l/16 the weights of nibble chunk g (bytes 32g..32g+31 of the
// 128): j < 4 the low nibbles of bytes 8j..8j+7 (sub-block 2g), j >= 4 the
// high nibbles of bytes 8(j-4)..+7 (sub-block 2g+1); its A lanes hold the same
// eight k. So each lane loads one contiguous 32-byte chunk per super-block,
// and the D lane's weight row is its own B row: d, dmin and the scales come
// from the header it loaded.
//
// The gated product (silu(W_gate x) * (W_up x), gate rows then up rows of
// one 2M-row matrix) runs the same way with a gate and an up row per lane,
// sharing the activation fragments, and applies the epilogue in fp32; its
// g and u are the stacked matrix's rows as the plain form sums them.
//
// Work: one workgroup of 8 waves per compute unit owns a contiguous range of
// 16-row tiles and stages the activations once (in chunks of super-blocks
// when a long row exceeds the LDS). The 8 waves split every tile's
// super-blocks; their sums meet in LDS and are added in wave order
// (deterministic). The next tile's weights are in flight while one is
// multiplied.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>

#include "q4_gemv_kernel.h"
#include "q4_internal.h"

namespace q4 {
namespace gemv {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));

constexpr int kMfmaWaves = 8;
constexpr int kMfmaSbMax = 4;     // most super-blocks per wave per tile and chunk
constexpr int kSbBytes = 144;     // Q4_K super-block
constexpr int kXRowPad = 16;      // bytes after each token's row of staged activations

// Two nibble codes (bytes B and B+1 of n) as the exact fp16 pair (sc q0, sc q1).
// A byte permute places each masked byte under the fp16 exponent of 1024:
// bits 0x64nn are 1024 + nn. A low nibble (nn = q) then takes one packed fma
// with sc and -1024 sc; a high nibble left in place (nn = 16 q) one with
// sc/16 and -64 sc. Both are exact: sc/16 is a multiple of 2^-4, every
// product and the result (an integer below 1024) fit fp16's 11 bits.
template <int B>
__device__ __forceinline__ uint32_t scaled_codes(uint32_t n, half2_t sc, half2_t off)
{
    constexpr uint32_t sel = B == 0 ? 0x04010400u : 0x04030402u;
    const half2_t c = __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(0x64646464u, n, sel));
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(c, sc, off));
}

// Eight codes from masked dwords a (codes 0..3) and b (4..7).
__device__ __forceinline__ half8 code8(uint32_t a, uint32_t b, half2_t sc, half2_t off)
{
    return __builtin_bit_cast(half8, u32x4{scaled_codes<0>(a, sc, off), scaled_codes<2>(a, sc, off),
                                           scaled_codes<0>(b, sc, off), scaled_codes<2>(b, sc, off)});
}

// Maximum over the 8 lanes of each aligned group of 8 (DPP: swap neighbours,
// swap pairs, mirror the halves of the 8).
__device__ __forceinline__ float max8(float v)
{
    const int b = __builtin_bit_cast(int, v);
    v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(b, b, 0xB1, 0xF, 0xF, false)));
    const int c = __builtin_bit_cast(int, v);
    v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(c, c, 0x4E, 0xF, 0xF, false)));
    const int d = __builtin_bit_cast(int, v);
    return fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(d, d, 0x141, 0xF, 0xF, false)));
}

// LDS. Wave v stages and reads its own columns v*SBW .. v*SBW + SBW - 1 (its
// super-blocks of the current chunk), so no wave waits for another's staging:
//   xs:  [n][8 SBW columns * 256] fp16, rows padded by kXRowPad bytes
//   scl: [8 SBW columns][16] fp32 2^e (zero for token slots n..15)
//   red: [2][gate, up][7 waves][64 lanes] f32x4, the waves' sums of a tile
struct MfmaLds {
    uint32_t xs, scl, red, total;
};

__host__ __device__ inline MfmaLds mfma_lds(int n, int sbw, bool glu = false)
{
    const uint32_t cols = static_cast<uint32_t>(kMfmaWaves) * static_cast<uint32_t>(sbw);
    MfmaLds l;
    l.xs = 0;
    l.scl = static_cast<uint32_t>(n) * (cols * 512u + kXRowPad);
    l.red = l.scl + cols * 64u;
    l.total = l.red + 2u * (glu ? 2u : 1u) * (kMfmaWaves - 1) * 64u * 16u;
    return l;
}

// GLU: the gated product. The weights have 2M rows (gate rows, then up
// rows); each tile's lanes load gate row r and up row M + r, the same
// activation fragments feed both, and y = silu(g) * u (one chunk only).
// ONE: every workgroup owns exactly one tile (the grid is the tile count).
template <int N, int SBW, bool GLU, bool ONE>
__global__ __launch_bounds__(64 * kMfmaWaves) void mfma_q4k_kernel(const uint8_t *__restrict__ w, uint32_t wbytes,
                                                                   const float *__restrict__ x, float *__restrict__ y,
                                                                   int M, int K, int CS)
{
    static_assert(N >= 1 && N <= 16 && SBW >= 1 && SBW <= kMfmaSbMax, "shape");
    constexpr int NR = GLU ? 2 : 1;  // weight rows per output row
    constexpr uint32_t xrow = kMfmaWaves * SBW * 512u + kXRowPad;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, col = lane & 15;
    const int ns = K / 256;
    const MfmaLds L = mfma_lds(N, SBW, GLU);
    const uint32_t wcol = static_cast<uint32_t>(wave) * SBW;  // this wave's first LDS column
    const int tiles = (M + 15) / 16;
    const int t0 = static_cast<int>(static_cast<int64_t>(blockIdx.x) * tiles / gridDim.x);
    const int t1 = static_cast<int>(static_cast<int64_t>(blockIdx.x + 1) * tiles / gridDim.x);
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(w, wbytes);
    const __amdgpu_buffer_rsrc_t xr =
        make_rsrc(x, static_cast<uint32_t>(static_cast<uint64_t>(N) * static_cast<uint64_t>(K) * 4u));
    const uint32_t row_bytes = static_cast<uint32_t>(ns) * kSbBytes;
    // This lane's A row in LDS: token col (slots past n repeat token 0).
    const uint32_t xa = static_cast<uint32_t>(col < N ? col : 0) * xrow + wcol * 512u + 128u * g;

    struct Set {
        u32x4 hd[NR][SBW], q0[NR][SBW], q1[NR][SBW];
    };
    // Super-blocks [s0, s0 + nsb) of tile t's row for this lane. Every one of
    // the SBW slots issues its loads (slots past nsb, rows past M and tiles
    // past t1 fetch nothing), so a set is always the same number of loads and
    // each wait covers exactly the loads it needs.
    auto load = [&](Set &st, int t, int s0, int nsb) __attribute__((always_inline)) {
        const int row = t * 16 + col;
        const bool live = t < t1 && row < M;
#pragma unroll
        for (int w = 0; w < NR; w++) {
            const uint32_t base = static_cast<uint32_t>(row + w * M) * row_bytes;
#pragma unroll
            for (int i = 0; i < SBW; i++) {
                const bool on = live && i < nsb;
                const uint32_t sbo = uniform(static_cast<uint32_t>(s0 + (i < nsb ? i : 0)) * kSbBytes);
                st.hd[w][i] = load16<0>(wr, on ? base : kNoFetch, sbo);
                st.q0[w][i] = load16<kNonTemporal>(wr, on ? base + 16u + 32u * g : kNoFetch, sbo);
                st.q1[w][i] = load16<kNonTemporal>(wr, on ? base + 32u + 32u * g : kNoFetch, sbo);
            }
        }
    };
    // One weight row's super-block decoded for the MFMAs: code scales and
    // offsets of its two sub-blocks, their mins broadcast, d and dmin.
    struct Dec {
        half2_t sc_a, off_a, sc_b, off_b;
        half8 bm_a, bm_b;
        float d, dmin;
    };
    auto decode = [&](const u32x4 &h) __attribute__((always_inline)) {
        // Sub-blocks 2g and 2g+1: their 6-bit fields sit in bytes
        // 2(g&1) and 2(g&1)+1 of the scale words.
        const uint32_t sh = (g & 1) << 4;
        const bool upper = g >= 2;
        const uint32_t w0 = h.y >> sh, w1 = h.z >> sh, w2 = h.w >> sh;
        const uint32_t sca = upper ? ((w2 & 15u) | (((w0 >> 6) & 3u) << 4)) : (w0 & 63u);
        const uint32_t scb = upper ? (((w2 >> 8) & 15u) | (((w0 >> 14) & 3u) << 4)) : ((w0 >> 8) & 63u);
        const uint32_t ma = upper ? (((w2 >> 4) & 15u) | (((w1 >> 6) & 3u) << 4)) : (w1 & 63u);
        const uint32_t mb = upper ? (((w2 >> 12) & 15u) | (((w1 >> 14) & 3u) << 4)) : ((w1 >> 8) & 63u);
        const _Float16 fa = static_cast<_Float16>(static_cast<float>(sca));
        const _Float16 fb = static_cast<_Float16>(static_cast<float>(scb));
        // Low nibbles: sc and -1024 sc; high nibbles in place: sc/16 and -64 sc.
        const _Float16 fb16 = fb * static_cast<_Float16>(0.0625f);
        const _Float16 oa = fa * static_cast<_Float16>(-1024.0f), ob = fb * static_cast<_Float16>(-64.0f);
        const _Float16 ha = static_cast<_Float16>(static_cast<float>(ma));
        const _Float16 hb = static_cast<_Float16>(static_cast<float>(mb));
        Dec e;
        e.sc_a = half2_t{fa, fa};
        e.off_a = half2_t{oa, oa};
        e.sc_b = half2_t{fb16, fb16};
        e.off_b = half2_t{ob, ob};
        e.bm_a = half8{ha, ha, ha, ha, ha, ha, ha, ha};
        e.bm_b = half8{hb, hb, hb, hb, hb, hb, hb, hb};
        e.d = half_lo(h.x);
        e.dmin = half_hi(h.x);
        return e;
    };
    // This wave's sums over its nsb super-blocks of one tile (the set's
    // weights against its own LDS columns), added to acc.
    auto partial = [&](const Set &st, int nsb, f32x4(&acc)[NR]) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < SBW; i++) {
            if (i < nsb) {
                Dec e[NR];
                uint32_t qw[NR][8];
#pragma unroll
                for (int w = 0; w < NR; w++) {
                    e[w] = decode(st.hd[w][i]);
                    const u32x4 a0 = st.q0[w][i], a1 = st.q1[w][i];
                    qw[w][0] = a0.x, qw[w][1] = a0.y, qw[w][2] = a0.z, qw[w][3] = a0.w;
                    qw[w][4] = a1.x, qw[w][5] = a1.y, qw[w][6] = a1.z, qw[w][7] = a1.w;
                }
                const uint8_t *xp = lds + xa + static_cast<uint32_t>(i) * 512u;
                f32x4 dq[NR], dm[NR];
#pragma unroll
                for (int w = 0; w < NR; w++) dq[w] = dm[w] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int j = 0; j < 8; j++) {
                    const half8 ax = *reinterpret_cast<const half8 *>(xp + 2 * (32 * (j >> 2) + 8 * (j & 3)));
#pragma unroll
                    for (int w = 0; w < NR; w++) {
                        const uint32_t qa = qw[w][2 * (j & 3)], qb = qw[w][2 * (j & 3) + 1];
                        const half8 bw = j < 4 ? code8(qa & 0x0F0F0F0Fu, qb & 0x0F0F0F0Fu, e[w].sc_a, e[w].off_a)
                                               : code8(qa & 0xF0F0F0F0u, qb & 0xF0F0F0F0u, e[w].sc_b, e[w].off_b);
                        dq[w] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ax, bw, dq[w], 0, 0, 0);
                        dm[w] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ax, j < 4 ? e[w].bm_a : e[w].bm_b, dm[w], 0, 0, 0);
                    }
                }
                const f32x4 sc4 = *reinterpret_cast<const f32x4 *>(lds + L.scl + ((wcol + i) * 16 + 4 * g) * 4);
#pragma unroll
                for (int w = 0; w < NR; w++)
#pragma unroll
                    for (int r = 0; r < 4; r++)
                        acc[w][r] = __builtin_fmaf(sc4[r], __builtin_fmaf(e[w].d, dq[w][r], -(e[w].dmin * dm[w][r])),
                                                   acc[w][r]);
            }
        }
    };
    // Tile t's sums of the workgroup, added in wave order through LDS
    // buffer buf (consecutive calls alternate buffers, so one barrier per
    // call suffices); wave 0 writes y, or adds to it (a later chunk).
    auto finish = [&](f32x4(&acc)[NR], int t, bool add, int buf) __attribute__((always_inline)) {
        f32x4 *red = reinterpret_cast<f32x4 *>(lds + L.red) + buf * NR * (kMfmaWaves - 1) * 64;
        if (wave > 0) {
#pragma unroll
            for (int w = 0; w < NR; w++) red[(w * (kMfmaWaves - 1) + wave - 1) * 64 + lane] = acc[w];
        }
        __syncthreads();
        if (wave == 0) {
#pragma unroll
            for (int w = 0; w < NR; w++)
#pragma unroll
                for (int v = 1; v < kMfmaWaves; v++) acc[w] += red[(w * (kMfmaWaves - 1) + v - 1) * 64 + lane];
            const int row = t * 16 + col;
            if (row < M) {
#pragma unroll
                for (int r = 0; r < 4; r++) {
                    const int tok = 4 * g + r;
                    if (tok < N) {
                        float *dst = y + static_cast<size_t>(tok) * M + row;
                        if constexpr (GLU)
                            *dst = silu_mul(acc[0][r], acc[1][r]);
                        else
                            *dst = add ? *dst + acc[0][r] : acc[0][r];
                    }
                }
            }
        }
    };

    // Staging of this wave's share [s0, s0 + nsb) of a chunk: pair p = t + N i
    // (token t, super-block s0 + i), 8 lanes per pair and 8 pairs per round.
    // Load j of a pair's 8 lanes reads the 128 bytes of sub-block j's
    // activations 4j.. (one cache line per load and pair), so lane l holds
    // elements 32j + 4l .. +3 for j < 8. R rounds per batch: a wave's whole
    // share in one batch where the registers allow (up to 3 rounds, 2 at
    // four super-blocks per wave).
    constexpr int R = SBW >= 4 ? 2 : ((N * SBW + 7) / 8 < 3 ? (N * SBW + 7) / 8 : 3);
    const int l8 = lane & 7, pj = lane >> 3;
    f32x4 v[R][8];
    auto stage_load = [&](int r0, int s0, int np) __attribute__((always_inline)) {
#pragma unroll
        for (int rr = 0; rr < R; rr++) {
            const int r = r0 + rr;
            if (8 * r >= np) {
                // No live pair in this round (uniform): no loads. The registers
                // are still set, so no earlier batch's values stay live.
#pragma unroll
                for (int j = 0; j < 8; j++) v[rr][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
                continue;
            }
            const int p = 8 * r + pj;
            const int t = p % N, i = p / N;
            const uint32_t off = p < np ? (static_cast<uint32_t>(t) * K + static_cast<uint32_t>(s0 + i) * 256u +
                                           4u * l8) * 4u
                                        : kNoFetch;
#pragma unroll
            for (int j = 0; j < 8; j++)
                v[rr][j] = __builtin_bit_cast(f32x4, load16<0>(xr, off == kNoFetch ? kNoFetch : off + 128u * j, 0));
        }
    };
    auto stage_convert = [&](int r0, int np) __attribute__((always_inline)) {
#pragma unroll
        for (int rr = 0; rr < R; rr++) {
            const int p = 8 * (r0 + rr) + pj;
            if (p < np) {
                const int t = p % N, i = p / N;
                float mx = 0.0f;
#pragma unroll
                for (int j = 0; j < 8; j++)
                    mx = fmaxf(mx, fmaxf(fmaxf(fabsf(v[rr][j].x), fabsf(v[rr][j].y)),
                                         fmaxf(fabsf(v[rr][j].z), fabsf(v[rr][j].w))));
                mx = max8(mx);
                // Largest magnitude into [2^14, 2^15): scale by 2^(14 - floor(log2(mx))).
                const int ex = static_cast<int>((__builtin_bit_cast(uint32_t, mx) >> 23) & 255u) - 127;
                const int shift = mx == 0.0f ? 0 : 14 - ex;
                uint8_t *dst = lds + L.xs + t * xrow + ((wcol + i) * 256 + 4 * l8) * 2;
#pragma unroll
                for (int j = 0; j < 8; j++) {
                    const f32x4 a = v[rr][j];
                    const half2_t h01 = {static_cast<_Float16>(__builtin_amdgcn_ldexpf(a.x, shift)),
                                         static_cast<_Float16>(__builtin_amdgcn_ldexpf(a.y, shift))};
                    const half2_t h23 = {static_cast<_Float16>(__builtin_amdgcn_ldexpf(a.z, shift)),
                                         static_cast<_Float16>(__builtin_amdgcn_ldexpf(a.w, shift))};
                    *reinterpret_cast<u32x2 *>(dst + 64 * j) =
                        u32x2{__builtin_bit_cast(uint32_t, h01), __builtin_bit_cast(uint32_t, h23)};
                }
                if (l8 == 0)
                    *reinterpret_cast<float *>(lds + L.scl + ((wcol + i) * 16 + t) * 4) =
                        __builtin_amdgcn_ldexpf(1.0f, -shift);
            }
        }
    };
    // Batches after the first.
    auto stage_rest = [&](int s0, int np) __attribute__((always_inline)) {
        for (int r0 = R; 8 * r0 < np; r0 += R) {
            stage_load(r0, s0, np);
            stage_convert(r0, np);
        }
    };
    // This wave's share of the chunk starting at super-block cb.
    auto share = [&](int cb, int &s0, int &nsb) __attribute__((always_inline)) {
        const int csz = ns - cb < CS ? ns - cb : CS;
        s0 = cb + wave * csz / kMfmaWaves;
        nsb = cb + (wave + 1) * csz / kMfmaWaves - s0;
    };

    // Token slots n..15 scale to zero in this wave's columns (never stored).
    for (int e = lane; e < 16 * SBW; e += 64)
        if ((e & 15) >= N) *reinterpret_cast<float *>(lds + L.scl + (wcol * 16 + e) * 4) = 0.0f;

    Set sa, sb;
    int s0, nsb;
    share(0, s0, nsb);
    // The first staging batch's loads go out ahead of the first tile's
    // weights: its conversion then waits for them alone, while the weights'
    // longer trip from HBM overlaps the staging.
    stage_load(0, s0, N * nsb);
    load(sa, t0, s0, nsb);
    stage_convert(0, N * nsb);
    stage_rest(s0, N * nsb);

    if constexpr (ONE) {
        // One tile: the sums carry over the chunks and meet once. The next
        // chunk's weights are in flight while one chunk is multiplied (its
        // activations are staged after, from L2; in flight across the
        // multiply they would not fit the registers). Each path is
        // straight-line and issues a fixed number of weight loads, so every
        // wait covers exactly the loads it needs.
        f32x4 acc[NR];
#pragma unroll
        for (int w = 0; w < NR; w++) acc[w] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        for (int cb = 0;;) {
            if (cb + CS >= ns) {
                partial(sa, nsb, acc);
                break;
            }
            int s1, n1;
            share(cb + CS, s1, n1);
            load(sb, t0, s1, n1);
            partial(sa, nsb, acc);
            stage_load(0, s1, N * n1);
            stage_convert(0, N * n1);
            stage_rest(s1, N * n1);
            cb += CS, s0 = s1, nsb = n1;
            if (cb + CS >= ns) {
                partial(sb, nsb, acc);
                break;
            }
            share(cb + CS, s1, n1);
            load(sa, t0, s1, n1);
            partial(sb, nsb, acc);
            stage_load(0, s1, N * n1);
            stage_convert(0, N * n1);
            stage_rest(s1, N * n1);
            cb += CS, s0 = s1, nsb = n1;
        }
        finish(acc, t0, false, 0);
    } else {
    // Several tiles: per chunk, the tiles with the next one's weights in
    // flight; a later chunk adds to y. Past the last tile no loads are
    // issued (a load that fetches nothing still costs the address unit a
    // pass over the wave); each path is straight-line, so its waits stay
    // exact.
    int buf = 0;
    auto one = [&](const Set &st, int t, bool add) __attribute__((always_inline)) {
        f32x4 acc[NR];
#pragma unroll
        for (int w = 0; w < NR; w++) acc[w] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        partial(st, nsb, acc);
        finish(acc, t, add, buf);
        buf ^= 1;
    };
    for (int cb = 0; cb < ns; cb += CS) {
        if (cb > 0) {
            share(cb, s0, nsb);
            stage_load(0, s0, N * nsb);
            load(sa, t0, s0, nsb);
            stage_convert(0, N * nsb);
            stage_rest(s0, N * nsb);
        }
        if constexpr (GLU) {
            // Two rows per lane: the straight-line paths below would keep more
            // registers live than the wave has, so past the last tile the
            // gated form issues loads that fetch nothing.
            for (int t = t0; t < t1; t += 2) {
                load(sb, t + 1, s0, nsb);
                one(sa, t, cb > 0);
                load(sa, t + 2, s0, nsb);
                if (t + 1 < t1) one(sb, t + 1, cb > 0);
            }
        } else {
            for (int t = t0; t < t1; t += 2) {
                if (t + 1 >= t1) {
                    one(sa, t, cb > 0);
                    break;
                }
                load(sb, t + 1, s0, nsb);
                one(sa, t, cb > 0);
                if (t + 2 >= t1) {
                    one(sb, t + 1, cb > 0);
                    break;
                }
                load(sa, t + 2, s0, nsb);
                one(sb, t + 1, cb > 0);
            }
        }
    }
    }
}

// The LDS opt-in above 64 KiB, once per kernel and device.
template <int N, int SBW, bool GLU, bool ONE>
int opt_in_lds(size_t lds, int budget)
{
    if (lds <= static_cast<size_t>(kMaxLdsBytes)) return Q4_OK;
    static std::atomic<int> opted[64];
    int dev = 0;
    if (hip_status(hipGetDevice(&dev)) != Q4_OK) return Q4_EHIP;
    if (dev < 0 || dev >= 64) return Q4_EUNSUPPORTED;
    if (!opted[dev].load(std::memory_order_acquire)) {
        const int st = hip_status(hipFuncSetAttribute(reinterpret_cast<const void *>(&mfma_q4k_kernel<N, SBW, GLU, ONE>),
                                                      hipFuncAttributeMaxDynamicSharedMemorySize, budget));
        if (st != Q4_OK) return st;
        opted[dev].store(1, std::memory_order_release);
    }
    return Q4_OK;
}

template <int N, int SBW, bool GLU>
int launch_mfma_sbw(const uint8_t *w, const float *x, float *y, int m, int k, int cs, size_t lds, int budget,
                    hipStream_t s, int cus, int groups_per_cu)
{
    if constexpr (GLU && SBW > 2) {
        return Q4_EUNSUPPORTED;  // the gated product keeps two rows' loads in flight: at most 2 per wave
    } else {
        const int tiles = (m + 15) / 16;
        const int cap = cus * (groups_per_cu > 0 ? groups_per_cu : 1);
        const unsigned grid = static_cast<unsigned>(tiles < cap ? tiles : cap);
        const uint32_t wbytes = static_cast<uint32_t>(q4_weight_bytes(Q4_FMT_Q4_K, GLU ? 2LL * m : m, k));
        // One tile per workgroup when the tiles fit the grid.
        if (static_cast<int>(grid) == tiles) {
            const int st = opt_in_lds<N, SBW, GLU, true>(lds, budget);
            if (st != Q4_OK) return st;
            hipLaunchKernelGGL((mfma_q4k_kernel<N, SBW, GLU, true>), dim3(grid), dim3(64 * kMfmaWaves), lds, s, w,
                               wbytes, x, y, m, k, cs);
        } else {
            const int st = opt_in_lds<N, SBW, GLU, false>(lds, budget);
            if (st != Q4_OK) return st;
            hipLaunchKernelGGL((mfma_q4k_kernel<N, SBW, GLU, false>), dim3(grid), dim3(64 * kMfmaWaves), lds, s, w,
                               wbytes, x, y, m, k, cs);
        }
        return hip_status(hipGetLastError());
    }
}

template <int N, bool GLU>
int launch_mfma(const uint8_t *w, const float *x, float *y, int m, int k, hipStream_t s, int cus, int groups_per_cu)
{
    const int ns = k / 256;
    // Chunks of at most 8 kMfmaSbMax super-blocks (four per wave per tile)
    // whose staged activations fit the LDS (the opt-in size above 64 KiB):
    // SBW, the most super-blocks per wave, sets the LDS columns.
    // The gated product takes rows of at most 16 super-blocks, in one chunk.
    if (GLU && ns > 2 * kMfmaWaves) return Q4_EUNSUPPORTED;
    int budget = kMaxLdsBytes;
    const int optin = device_lds_optin();
    int sbw = (ns + kMfmaWaves - 1) / kMfmaWaves;
    if (sbw > kMfmaSbMax) sbw = kMfmaSbMax;
    if (mfma_lds(N, sbw, GLU).total > static_cast<uint32_t>(budget) && optin > budget) budget = optin;
    while (sbw > 1 && mfma_lds(N, sbw, GLU).total > static_cast<uint32_t>(budget)) sbw--;
    if (mfma_lds(N, sbw, GLU).total > static_cast<uint32_t>(budget)) return Q4_EUNSUPPORTED;
    const int chunks = (ns + kMfmaWaves * sbw - 1) / (kMfmaWaves * sbw);
    if (GLU && chunks > 1) return Q4_EUNSUPPORTED;
    const int cs = (ns + chunks - 1) / chunks;  // even chunks
    sbw = (cs + kMfmaWaves - 1) / kMfmaWaves;
    const size_t lds = mfma_lds(N, sbw, GLU).total;
    switch (sbw) {
    case 1: return launch_mfma_sbw<N, 1, GLU>(w, x, y, m, k, cs, lds, budget, s, cus, groups_per_cu);
    case 2: return launch_mfma_sbw<N, 2, GLU>(w, x, y, m, k, cs, lds, budget, s, cus, groups_per_cu);
    case 3: return launch_mfma_sbw<N, 3, GLU>(w, x, y, m, k, cs, lds, budget, s, cus, groups_per_cu);
    default: return launch_mfma_sbw<N, 4, GLU>(w, x, y, m, k, cs, lds, budget, s, cus, groups_per_cu);
    }
}

template <bool GLU>
int dispatch_mfma_glu(const uint8_t *w, const float *x, float *y, int m, int k, int n, hipStream_t s, int cus,
                      int groups_per_cu)
{
    switch (n) {
    case 1: return launch_mfma<1, GLU>(w, x, y, m, k, s, cus, groups_per_cu);
    case 2: return launch_mfma<2, GLU>(w, x, y, m, k, s, cus, groups_per_cu);
    case 3: return launch_mfma<3, GLU>(w, x, y, m, k, s, cus, groups_per_cu);
    case 4: return launch_mfma<4, GLU>(w, x, y, m, k, s, cus, groups_per_cu);
    case 5: return launch_mfma<5, GLU>(w, x, y, m, k, s, cus, groups_per_cu);
    case 6: return launch_mfma<6, GLU>(w, x, y, m, k, s, cus, groups_per_cu);
    case 7: return launch_mfma<7, GLU>(w, x, y, m, k, s, cus, groups_per_cu);
    case 8: return launch_mfma<8, GLU>(w, x, y, m, k, s, cus, groups_per_cu);
    default: return Q4_EUNSUPPORTED;
    }
}

int dispatch_mfma(const uint8_t *w, const float *x, float *y, int m, int k, int n, hipStream_t s, int cus,
                  int groups_per_cu, bool glu)
{
    return glu ? dispatch_mfma_glu<true>(w, x, y, m, k, n, s, cus, groups_per_cu)
               : dispatch_mfma_glu<false>(w, x, y, m, k, n, s, cus, groups_per_cu);
}

}  // namespace gemv
}  // namespace q4
