// Prefill product Y = bf16(W_hat) X for 4-bit block-quantized W on gfx950.
//
// Method (Llamas on the Web, technical summary, Methodology section 3,
// "integrated dequantization"): for the matrix-matrix product the quantized
// blocks are loaded, dequantized into shared memory and reused; on gfx950 the
// reuse is by bf16 matrix-core instructions (v_mfma_f32_16x16x32_bf16, fp32
// accumulation), since prefill is a dense contraction.
//
// Work decomposition: a workgroup of 4 waves computes a TM (weight rows) x TN
// (tokens) tile of Y over all of K, in chunks of KC along K.
//   * Weights: each chunk's TM x KC quantized tile is dequantized exactly in
//     fp32 ((q-8)*d, or d*sc*q - dmin*m for Q4_K), rounded to bf16 (RNE) and
//     written to LDS once; all four waves read it as MFMA A operands, so each
//     dequantized weight is reused across the whole token tile. The packed
//     tile of chunk c+1 is loaded into registers while chunk c is multiplied.
//   * Activations: every wave owns TN/4 tokens, so its bf16 X fragments go
//     straight from memory into registers in the MFMA B layout (no LDS),
//     through a ring of XD 32-wide k slices that is refilled as it is
//     consumed, so XD slices of loads are in flight behind the MFMAs.
//   * Loads are raw buffer loads and are all issued unconditionally: rows past
//     M, tokens past N and k past K read zeros (out-of-range offsets), so the
//     last chunk is padded with zero products and no branch sits between
//     slices, which keeps the compiler's wait counting exact.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>

#include "q4_internal.h"

namespace q4 {
namespace gemm {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBufferWord3 = 0x00020000; // raw 32-bit buffer descriptor, gfx9 family
// A lane offset past every descriptor's range (operands are below 2 GiB): the
// load returns zeros without a memory request.
constexpr uint32_t kNoFetch = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), static_cast<short>(0), static_cast<int>(bytes),
                                             kBufferWord3);
}

__device__ __forceinline__ float half_bits_to_float(uint32_t h)
{
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(h & 0xFFFFu)));
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Two fp32 values rounded to bf16 (RNE) in one dword (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float a, float b)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// Nibbles of bytes K and K+1 of `n` (each byte already masked to its nibble q)
// as the exact fp16 pair (q + 1024 + add): a byte permute places each nibble
// under the fp16 exponent of 1024 (bits 0x64nn = 1024 + q), then one packed
// fp16 add. With add = -1032 the pair is q - 8, with add = -1024 it is q.
template <int K>
__device__ __forceinline__ half2_t nibble_pair(uint32_t n, half2_t add)
{
    constexpr uint32_t sel = K == 0 ? 0x04010400u : 0x04030402u;  // bytes {K, 0x64, K+1, 0x64}
    return __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(0x64646464u, n, sel)) + add;
}

// Eight weights from the masked nibble dwords n0 (elements 0..3) and n1
// (4..7): value(q) for each, as 8 bf16 in 16 bytes.
template <class V>
__device__ __forceinline__ u32x4 eight(uint32_t n0, uint32_t n1, half2_t add, V value)
{
    const half2_t p0 = nibble_pair<0>(n0, add), p1 = nibble_pair<2>(n0, add);
    const half2_t p2 = nibble_pair<0>(n1, add), p3 = nibble_pair<2>(n1, add);
    return u32x4{pack_bf16(value(p0[0]), value(p0[1])), pack_bf16(value(p1[0]), value(p1[1])),
                 pack_bf16(value(p2[0]), value(p2[1])), pack_bf16(value(p3[0]), value(p3[1]))};
}

// ---- format policies ------------------------------------------------------------
// A chunk item is 16 weights of one row: two nibble dwords whose low nibbles
// are chunk elements lo..lo+7 and whose high nibbles are hi..hi+7. It is
// written to LDS as two 16-byte runs of bf16.

struct GemmQ4_0 {
    static constexpr int kFormat = Q4_FMT_Q4_0;
    static constexpr int kRingVgprs = 128;  // activation ring budget (Items are 3 VGPRs)
    __device__ static uint32_t scale_plane(uint64_t rows, uint64_t k) { return static_cast<uint32_t>(rows * k / 2u); }
    struct Item {
        u32x2 q;     // 8 nibble bytes
        uint32_t d;  // fp16 scale bits
    };
    // Item it (0 .. KC/16-1) of chunk s (KC weights per row): block
    // s*KC/32 + it/2 of the row, nibble bytes 8*(it%2) .. +7. Items of a
    // block past the row's end, or of a row past M, read zeros (d = 0, so
    // they dequantize to zero).
    template <int KC>
    __device__ static void load(Item &g, const uint8_t *w, uint32_t wbytes, uint32_t scale_plane, uint32_t nu,
                                uint32_t row, bool row_ok, int s, int it)
    {
        const __amdgpu_buffer_rsrc_t r = make_rsrc(w, wbytes);
        const uint32_t ub = static_cast<uint32_t>(s * (KC / 32) + (it >> 1));
        const uint32_t blk = row * nu + ub;
        const bool live = row_ok && ub < nu;
        g.q = __builtin_bit_cast(
            u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, live ? blk * 16u + 8u * static_cast<uint32_t>(it & 1) : kNoFetch,
                                                        0, 0));
        g.d = __builtin_amdgcn_raw_buffer_load_b16(r, live ? scale_plane + blk * 2u : kNoFetch, 0, 0);
    }
    __device__ static int lo(int it) { return 32 * (it >> 1) + 8 * (it & 1); }
    __device__ static int hi(int it) { return lo(it) + 16; }
    // (q - 8) * d: the fp16 code q - 8 times the fp16 scale is exact in fp32,
    // so the only rounding is the final one to bf16.
    template <int KC>
    __device__ static void dequant(const Item &g, int /*s*/, int /*it*/, u32x4 &vlo, u32x4 &vhi)
    {
        const float d = half_bits_to_float(g.d);
        const half2_t add = {static_cast<_Float16>(-1032.0f), static_cast<_Float16>(-1032.0f)};
        // Written as an fma with a zero addend so the fp16 operand feeds v_fma_mix_f32 directly
        // (the product is exact, so the fma returns it unchanged; q - 8 is never -0).
        const auto value = [d](_Float16 c) { return __builtin_fmaf(static_cast<float>(c), d, 0.0f); };
        vlo = eight(g.q.x & 0x0F0F0F0Fu, g.q.y & 0x0F0F0F0Fu, add, value);
        vhi = eight((g.q.x >> 4) & 0x0F0F0F0Fu, (g.q.y >> 4) & 0x0F0F0F0Fu, add, value);
    }
};

// Q8_0: an item is 16 consecutive weights of one block, half h = it & 1 of
// block it / 2: code bytes 16h .. 16h+15 (elements lo .. lo+7 and hi .. hi+7,
// hi = lo + 8). Codes become exact fp16 values by the byte-permute trick
// (offset by 128 under the exponent of 1024, then -1152).
struct GemmQ8_0 {
    static constexpr int kFormat = Q4_FMT_Q8_0;
    static constexpr int kRingVgprs = 64;  // activation ring budget (Items are 5 VGPRs)
    __device__ static uint32_t scale_plane(uint64_t rows, uint64_t k) { return static_cast<uint32_t>(rows * k); }
    struct Item {
        u32x4 q;     // 16 code bytes
        uint32_t d;  // fp16 scale bits
    };
    template <int KC>
    __device__ static void load(Item &g, const uint8_t *w, uint32_t wbytes, uint32_t scale_plane, uint32_t nu,
                                uint32_t row, bool row_ok, int s, int it)
    {
        const __amdgpu_buffer_rsrc_t r = make_rsrc(w, wbytes);
        const uint32_t ub = static_cast<uint32_t>(s * (KC / 32) + (it >> 1));
        const uint32_t blk = row * nu + ub;
        const bool live = row_ok && ub < nu;
        g.q = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, live ? blk * 32u + 16u * static_cast<uint32_t>(it & 1) : kNoFetch,
                                                         0, 0));
        g.d = __builtin_amdgcn_raw_buffer_load_b16(r, live ? scale_plane + blk * 2u : kNoFetch, 0, 0);
    }
    __device__ static int lo(int it) { return 32 * (it >> 1) + 16 * (it & 1); }
    __device__ static int hi(int it) { return lo(it) + 8; }
    // q * d: exact in fp32 (8 + 11 significant bits); the only rounding is to bf16.
    template <int KC>
    __device__ static void dequant(const Item &g, int /*s*/, int /*it*/, u32x4 &vlo, u32x4 &vhi)
    {
        const float d = half_bits_to_float(g.d);
        const half2_t add = {static_cast<_Float16>(-1152.0f), static_cast<_Float16>(-1152.0f)};
        const auto value = [d](_Float16 c) { return __builtin_fmaf(static_cast<float>(c), d, 0.0f); };
        vlo = eight(g.q.x ^ 0x80808080u, g.q.y ^ 0x80808080u, add, value);
        vhi = eight(g.q.z ^ 0x80808080u, g.q.w ^ 0x80808080u, add, value);
    }
};

// Q1_0: an item is 16 consecutive weights of one block, half h = it & 1 of
// block it / 2: code bits 16h .. 16h+15 (elements lo .. lo+7 and hi .. hi+7,
// hi = lo + 8), loaded as one 16-bit half of the code word. A weight is
// +d or -d, so its bf16 is bf16(d) with the sign flipped where the code is 0.
struct GemmQ1_0 {
    static constexpr int kFormat = Q4_FMT_Q1_0;
    static constexpr int kRingVgprs = 128;  // activation ring budget (Items are 2 VGPRs)
    __device__ static uint32_t scale_plane(uint64_t rows, uint64_t k) { return static_cast<uint32_t>(rows * k / 8u); }
    struct Item {
        uint32_t q;  // 16 code bits (low half)
        uint32_t d;  // fp16 scale bits
    };
    template <int KC>
    __device__ static void load(Item &g, const uint8_t *w, uint32_t wbytes, uint32_t scale_plane, uint32_t nu,
                                uint32_t row, bool row_ok, int s, int it)
    {
        const __amdgpu_buffer_rsrc_t r = make_rsrc(w, wbytes);
        const uint32_t ub = static_cast<uint32_t>(s * (KC / 32) + (it >> 1));
        const uint32_t blk = row * nu + ub;
        const bool live = row_ok && ub < nu;
        g.q = __builtin_amdgcn_raw_buffer_load_b16(r, live ? blk * 4u + 2u * static_cast<uint32_t>(it & 1) : kNoFetch,
                                                   0, 0);
        g.d = __builtin_amdgcn_raw_buffer_load_b16(r, live ? scale_plane + blk * 2u : kNoFetch, 0, 0);
    }
    __device__ static int lo(int it) { return 32 * (it >> 1) + 16 * (it & 1); }
    __device__ static int hi(int it) { return lo(it) + 8; }
    // Eight weights from code bits j0 .. j0+7 of the half: pairs of bf16(d)
    // with the sign flipped by the inverted codes (a flip, not a set, so a
    // negative scale in a hand-built buffer still gives (2b - 1) d).
    __device__ static u32x4 eight_signs(uint32_t neg, uint32_t dd, int j0)
    {
        u32x4 v;
#pragma unroll
        for (int p = 0; p < 4; p++) {
            const uint32_t a = neg >> (j0 + 2 * p);
            v[p] = dd ^ (((a << 15) & 0x8000u) | ((a << 30) & 0x80000000u));
        }
        return v;
    }
    // bf16_rne(+-d) = +-bf16_rne(d): the only rounding is that of d.
    template <int KC>
    __device__ static void dequant(const Item &g, int /*s*/, int /*it*/, u32x4 &vlo, u32x4 &vhi)
    {
        const float d = half_bits_to_float(g.d);
        const uint32_t dd = pack_bf16(d, d);
        const uint32_t neg = ~g.q;
        vlo = eight_signs(neg, dd, 0);
        vhi = eight_signs(neg, dd, 8);
    }
};

// Q2_K: an item is two 8-element runs of one super-block that share 8 code
// bytes: w16 = it % 16 of super-block s*KC/256 + it/16 gives half h = w16/8,
// run pair p = (w16/4) % 2 and byte group i = w16 % 4: code bytes 32h + 8i ..
// +7, whose bit pairs 4p and 4p+2 hold runs j = 2p and 2p+1 (elements
// 128h + 32j + 8i .. +7). Run j lies in sub-block 8h + 2j + (i >= 2).
struct GemmQ2_K {
    static constexpr int kFormat = Q4_FMT_Q2_K;
    static constexpr int kRingVgprs = 64;  // activation ring budget (Items are 7 VGPRs)
    __device__ static uint32_t scale_plane(uint64_t rows, uint64_t k) { return static_cast<uint32_t>(rows * k / 4u); }
    struct Item {
        u32x2 q;      // 8 code bytes
        u32x4 sc;     // the super-block's 16 scale bytes
        uint32_t dd;  // fp16 d | fp16 dmin << 16
    };
    template <int KC>
    __device__ static void load(Item &g, const uint8_t *w, uint32_t wbytes, uint32_t scale_plane, uint32_t nu,
                                uint32_t row, bool row_ok, int s, int it)
    {
        const __amdgpu_buffer_rsrc_t r = make_rsrc(w, wbytes);
        const uint32_t ns = nu >> 3;
        const uint32_t sbr = static_cast<uint32_t>(s * (KC / 256) + (it >> 4));
        const bool live = row_ok && sbr < ns;
        const uint32_t sb = row * ns + sbr;
        const uint32_t w16 = static_cast<uint32_t>(it & 15);
        const uint32_t byte = 32u * (w16 >> 3) + 8u * (w16 & 3u);
        g.q = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, live ? sb * 64u + byte : kNoFetch, 0, 0));
        g.sc = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, live ? scale_plane + sb * 16u : kNoFetch,
                                                                                0, 0));
        g.dd = __builtin_amdgcn_raw_buffer_load_b32(r, live ? scale_plane + scale_plane / 4u + sb * 4u : kNoFetch, 0, 0);
    }
    __device__ static int lo(int it)
    {
        const int w16 = it & 15;
        return 256 * (it >> 4) + 128 * (w16 >> 3) + 64 * ((w16 >> 2) & 1) + 8 * (w16 & 3);
    }
    __device__ static int hi(int it) { return lo(it) + 32; }
    // (d*sc)*q - dmin*m: (d*sc)*q is exact in fp32, so the fma rounds the exact
    // difference once, as the format's definition does.
    template <int KC>
    __device__ static void dequant(const Item &g, int /*s*/, int it, u32x4 &vlo, u32x4 &vhi)
    {
        const int w16 = it & 15;
        const int h = w16 >> 3, p = (w16 >> 2) & 1, c = (w16 & 3) >> 1;
        const float d = half_bits_to_float(g.dd), dmin = half_bits_to_float(g.dd >> 16);
        const auto scale_byte = [&](int j) {
            const int b = 8 * h + 2 * j + c;
            const uint32_t word = b < 4 ? g.sc.x : b < 8 ? g.sc.y : b < 12 ? g.sc.z : g.sc.w;
            return (word >> (8 * (b & 3))) & 0xFFu;
        };
        const half2_t add = {static_cast<_Float16>(-1024.0f), static_cast<_Float16>(-1024.0f)};
        const int ja = 2 * p, jb = 2 * p + 1;
        const uint32_t sa = scale_byte(ja), sbb = scale_byte(jb);
        const float stepa = d * static_cast<float>(sa & 15u), offa = -(dmin * static_cast<float>(sa >> 4));
        const float stepb = d * static_cast<float>(sbb & 15u), offb = -(dmin * static_cast<float>(sbb >> 4));
        vlo = eight((g.q.x >> (2 * ja)) & 0x03030303u, (g.q.y >> (2 * ja)) & 0x03030303u, add,
                    [=](_Float16 q) { return __builtin_fmaf(stepa, static_cast<float>(q), offa); });
        vhi = eight((g.q.x >> (2 * jb)) & 0x03030303u, (g.q.y >> (2 * jb)) & 0x03030303u, add,
                    [=](_Float16 q) { return __builtin_fmaf(stepb, static_cast<float>(q), offb); });
    }
};

struct GemmQ4_K {
    static constexpr int kFormat = Q4_FMT_Q4_K;
    static constexpr int kRingVgprs = 64;  // activation ring budget (Items are 6 VGPRs)
    __device__ static uint32_t scale_plane(uint64_t, uint64_t) { return 0; }  // headers are in the super-blocks
    struct Item {
        u32x2 q;  // 8 nibble bytes
        u32x4 h;  // super-block header: d, dmin, 12 scale bytes
    };
    // Chunk s covers 64-weight nibble groups s*KC/64 .. of the row (4 groups
    // of 32 bytes per super-block); item it is bytes 8*(it%4) .. +7 of group
    // s*KC/64 + it/4. Byte i of a group c holds elements 64c+i (sub-block 2c)
    // and 64c+32+i (sub-block 2c+1). Items past the row's end, or of a row
    // past M, read zeros (d = dmin = 0).
    template <int KC>
    __device__ static void load(Item &g, const uint8_t *w, uint32_t wbytes, uint32_t /*scale_plane*/, uint32_t nu,
                                uint32_t row, bool row_ok, int s, int it)
    {
        const __amdgpu_buffer_rsrc_t r = make_rsrc(w, wbytes);
        const uint32_t grp = static_cast<uint32_t>(s * (KC / 64) + (it >> 2));
        const bool live = row_ok && (grp >> 2) < (nu >> 3);
        const uint32_t base = live ? (row * (nu >> 3) + (grp >> 2)) * 144u : kNoFetch;
        g.h = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, base, 0, 0));
        g.q = __builtin_bit_cast(
            u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, base + 16u + 32u * (grp & 3u) + 8u * static_cast<uint32_t>(it & 3),
                                                        0, 0));
    }
    __device__ static int lo(int it) { return 64 * (it >> 2) + 8 * (it & 3); }
    __device__ static int hi(int it) { return lo(it) + 32; }
    // d*sc*q - dmin*m: d*sc*q is exact in fp32 (<= 21 bits), so the fma rounds
    // the exact difference once, as the format's definition does.
    template <int KC>
    __device__ static void dequant(const Item &g, int s, int it, u32x4 &vlo, u32x4 &vhi)
    {
        // Sub-blocks a = 2c, b = 2c+1 of group c (within the super-block);
        // their 6-bit fields sit in bytes 2(c&1), 2(c&1)+1 of the scale words.
        const uint32_t c = static_cast<uint32_t>(s * (KC / 64) + (it >> 2)) & 3u;
        const uint32_t sh = (c & 1u) << 4;
        const uint32_t s0 = g.h.y >> sh, s1 = g.h.z >> sh, s2 = g.h.w >> sh;
        const bool upper = c >= 2;
        const uint32_t sca = upper ? ((s2 & 15u) | (((s0 >> 6) & 3u) << 4)) : (s0 & 63u);
        const uint32_t scb = upper ? (((s2 >> 8) & 15u) | (((s0 >> 14) & 3u) << 4)) : ((s0 >> 8) & 63u);
        const uint32_t ma = upper ? (((s2 >> 4) & 15u) | (((s1 >> 6) & 3u) << 4)) : (s1 & 63u);
        const uint32_t mb = upper ? (((s2 >> 12) & 15u) | (((s1 >> 14) & 3u) << 4)) : ((s1 >> 8) & 63u);
        const float d = half_bits_to_float(g.h.x), dmin = half_bits_to_float(g.h.x >> 16);
        const float stepa = d * static_cast<float>(sca), stepb = d * static_cast<float>(scb);
        const float offa = -(dmin * static_cast<float>(ma)), offb = -(dmin * static_cast<float>(mb));
        const half2_t add = {static_cast<_Float16>(-1024.0f), static_cast<_Float16>(-1024.0f)};
        vlo = eight(g.q.x & 0x0F0F0F0Fu, g.q.y & 0x0F0F0F0Fu, add,
                    [=](_Float16 q) { return __builtin_fmaf(stepa, static_cast<float>(q), offa); });
        vhi = eight((g.q.x >> 4) & 0x0F0F0F0Fu, (g.q.y >> 4) & 0x0F0F0F0Fu, add,
                    [=](_Float16 q) { return __builtin_fmaf(stepb, static_cast<float>(q), offb); });
    }
};

// ---- the kernel ---------------------------------------------------------------------
// MFMA 16x16x32 operand layout (wave64): A (16 rows x 32 k): lane l holds row
// l%16, k = 8(l/16)..8(l/16)+7; B (32 k x 16 cols): lane l holds column
// l%16, the same k range; D (16 x 16): lane l holds rows 4(l/16)..+3 of
// column l%16. Rows are weight rows, columns are tokens.

template <class F, int TM, int TN, int KC>
__global__ __launch_bounds__(256) void gemm_kernel(const uint8_t *__restrict__ w, uint32_t wbytes,
                                                   const uint16_t *__restrict__ x, float *__restrict__ y, int M,
                                                   int K, int N)
{
    constexpr int FM = TM / 16;              // A fragments (16-row blocks) per wave
    constexpr int WN = TN / 4;               // tokens per wave
    constexpr int FN = WN / 16;              // B fragments per wave
    constexpr int SPC = KC / 32;             // 32-wide k slices per chunk
    constexpr int XR = F::kRingVgprs / (4 * FN);
    constexpr int XD = SPC < XR ? SPC : XR;  // depth of the activation ring, in slices
    constexpr int IPR = KC / 16;             // weight items (16 weights) per row per chunk
    constexpr int WI = TM * IPR / 256;       // weight items per thread per chunk
    constexpr int kLdsRow = KC + 8;          // bf16 per LDS row (padding staggers banks)
    static_assert(WI >= 1 && FN >= 1 && TM * IPR % 256 == 0 && XD >= 1 && SPC % XD == 0, "bad tile");
    extern __shared__ __attribute__((aligned(16))) __bf16 ws[];  // TM x kLdsRow

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int r0 = blockIdx.x * TM;
    const int t0 = blockIdx.y * TN;
    const uint32_t nu = static_cast<uint32_t>(K / 32);
    const uint32_t scale_plane = F::scale_plane(static_cast<uint64_t>(M), static_cast<uint64_t>(K));
    const int C = (K + KC - 1) / KC;
    const __amdgpu_buffer_rsrc_t xr =
        make_rsrc(x, static_cast<uint32_t>(static_cast<uint64_t>(N) * static_cast<uint64_t>(K) * 2u));
    // This lane's k offset within a 32-slice, and the byte offset of its
    // token row for each B fragment (a token past N lies past the buffer).
    const int ktok = 8 * (lane >> 4);
    uint32_t xrow[FN];
#pragma unroll
    for (int fn = 0; fn < FN; fn++)
        xrow[fn] = (static_cast<uint32_t>(t0 + wave * WN + 16 * fn + (lane & 15)) * static_cast<uint32_t>(K) +
                    static_cast<uint32_t>(ktok)) * 2u;

    f32x4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; i++)
#pragma unroll
        for (int j = 0; j < FN; j++) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    typename F::Item gi[WI];
    bf16x8 xring[XD][FN];

    auto load_w = [&](int c) {
#pragma unroll
        for (int i = 0; i < WI; i++) {
            const int it = tid + 256 * i;
            const int row = r0 + it / IPR;
            F::template load<KC>(gi[i], w, wbytes, scale_plane, nu, static_cast<uint32_t>(row), row < M, c, it % IPR);
        }
    };
    // Global slice g (k = 32g ..) into ring slot j; past K: zeros, no fetch.
    auto load_x = [&](int j, int g) {
        const bool live = 32 * g < K;
#pragma unroll
        for (int fn = 0; fn < FN; fn++)
            xring[j][fn] = __builtin_bit_cast(
                bf16x8, __builtin_amdgcn_raw_buffer_load_b128(xr, live ? xrow[fn] + 64u * static_cast<uint32_t>(g) : kNoFetch,
                                                              0, 0));
    };
    auto write_w = [&](int c) {
#pragma unroll
        for (int i = 0; i < WI; i++) {
            const int it = tid + 256 * i;
            const int row = it / IPR, iw = it % IPR;
            u32x4 vlo, vhi;
            F::template dequant<KC>(gi[i], c, iw, vlo, vhi);
            *reinterpret_cast<u32x4 *>(&ws[row * kLdsRow + F::lo(iw)]) = vlo;
            *reinterpret_cast<u32x4 *>(&ws[row * kLdsRow + F::hi(iw)]) = vhi;
        }
    };

    // Issue order W(c) then X is the same before the loop and at every chunk
    // boundary, so each wait below is for exactly the loads it needs.
    load_w(0);
    __builtin_amdgcn_sched_barrier(0);  // keep W(0) ahead of the ring in issue order
#pragma unroll
    for (int j = 0; j < XD; j++) load_x(j, j);
    for (int c = 0; c < C; c++) {
        if (c > 0) __syncthreads();  // every wave is done with chunk c-1 in LDS
        write_w(c);
        __syncthreads();
        load_w(c + 1);  // past the last chunk: no fetch, never used
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int s0 = 0; s0 < SPC; s0 += XD) {
#pragma unroll
            for (int j = 0; j < XD; j++) {
                const int kk = s0 + j;
                bf16x8 a[FM];
#pragma unroll
                for (int fm = 0; fm < FM; fm++)
                    a[fm] = *reinterpret_cast<const bf16x8 *>(&ws[(16 * fm + (lane & 15)) * kLdsRow + 32 * kk + ktok]);
#pragma unroll
                for (int fm = 0; fm < FM; fm++)
#pragma unroll
                    for (int fn = 0; fn < FN; fn++)
                        acc[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[fm], xring[j][fn], acc[fm][fn], 0, 0, 0);
                load_x(j, c * SPC + kk + XD);
            }
        }
    }

    // Store: lane holds rows 4(l/16)..+3 of token column l%16 of each 16x16 tile.
#pragma unroll
    for (int fm = 0; fm < FM; fm++) {
        const int row = r0 + 16 * fm + 4 * (lane >> 4);
#pragma unroll
        for (int fn = 0; fn < FN; fn++) {
            const int tok = t0 + wave * WN + 16 * fn + (lane & 15);
            if (tok >= N) continue;
            float *dst = y + static_cast<size_t>(tok) * M + row;
            if (row + 3 < M && (reinterpret_cast<uintptr_t>(dst) & 15) == 0) {
                *reinterpret_cast<f32x4 *>(dst) = acc[fm][fn];
            } else {
#pragma unroll
                for (int r = 0; r < 4; r++)
                    if (row + r < M) dst[r] = acc[fm][fn][r];
            }
        }
    }
}

template <class F, int TM, int TN, int KC>
int launch_tile(const void *w, const uint16_t *x, float *y, int64_t m, int64_t k, int64_t n, hipStream_t s)
{
    constexpr size_t lds = static_cast<size_t>(TM) * (KC + 8) * 2;
    if constexpr (lds > 65536) {
        // Above 64 KB a kernel must opt in to its dynamic LDS size, once per device.
        static std::atomic<int> opted[64];
        int dev = 0;
        if (hip_status(hipGetDevice(&dev)) != Q4_OK) return Q4_EHIP;
        if (dev < 0 || dev >= 64) return Q4_EUNSUPPORTED;
        if (!opted[dev].load(std::memory_order_acquire)) {
            const int st = hip_status(hipFuncSetAttribute(reinterpret_cast<const void *>(&gemm_kernel<F, TM, TN, KC>),
                                                          hipFuncAttributeMaxDynamicSharedMemorySize,
                                                          static_cast<int>(lds)));
            if (st != Q4_OK) return st;
            opted[dev].store(1, std::memory_order_release);
        }
    }
    const uint32_t wbytes = static_cast<uint32_t>(q4_weight_bytes(F::kFormat, m, k));
    const dim3 grid(static_cast<unsigned>((m + TM - 1) / TM), static_cast<unsigned>((n + TN - 1) / TN));
    hipLaunchKernelGGL((gemm_kernel<F, TM, TN, KC>), grid, dim3(256), lds, s, static_cast<const uint8_t *>(w), wbytes,
                       x, y, static_cast<int>(m), static_cast<int>(k), static_cast<int>(n));
    return hip_status(hipGetLastError());
}

// Tile geometries: (rows, tokens, K per chunk). LDS per workgroup is
// rows x (chunk + 8) x 2 bytes (16 KB .. 66 KB here).
#define Q4_GEMM_TILES(X) \
    X(16, 64, 512)       \
    X(16, 64, 1024)      \
    X(32, 64, 256)       \
    X(32, 64, 512)       \
    X(32, 64, 1024)      \
    X(32, 128, 512)      \
    X(64, 64, 256)       \
    X(64, 64, 512)

template <class F>
int launch_geometry(int tm, int tn, int kc, const void *w, const uint16_t *x, float *y, int64_t m, int64_t k,
                    int64_t n, hipStream_t s)
{
#define Q4_TILE_CASE(A, B, C) \
    if (tm == A && tn == B && kc == C) return launch_tile<F, A, B, C>(w, x, y, m, k, n, s);
    Q4_GEMM_TILES(Q4_TILE_CASE)
#undef Q4_TILE_CASE
    return Q4_EUNSUPPORTED;
}

template <class F>
int launch_fmt(const void *w, const uint16_t *x, float *y, int64_t m, int64_t k, int64_t n, hipStream_t s, int cus)
{
    // From a sweep of the instantiated geometries on gfx950 at the SmolLM2-360M
    // layer shapes x 512 tokens: 32 x 64 tiles with 256-wide chunks, 16-row
    // tiles for short Q4_0 matrices (more workgroups in flight), and 64-row
    // tiles once the 32 x 64 grid exceeds two workgroups per compute unit.
    const int64_t tiles = ((m + 31) / 32) * ((n + 63) / 64);
    if (tiles > 2LL * cus) return launch_geometry<F>(64, 64, 256, w, x, y, m, k, n, s);
    if (F::kFormat == Q4_FMT_Q4_0 && m <= 512) return launch_geometry<F>(16, 64, 512, w, x, y, m, k, n, s);
    return launch_geometry<F>(32, 64, 256, w, x, y, m, k, n, s);
}

}  // namespace gemm

int launch_gemm(int fmt, const void *w, const uint16_t *x, float *y, int64_t m, int64_t k, int64_t n, void *stream)
{
    const int cus = device_cus();
    if (cus <= 0) return Q4_EHIP;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (fmt == Q4_FMT_Q4_0) return gemm::launch_fmt<gemm::GemmQ4_0>(w, x, y, m, k, n, s, cus);
    if (fmt == Q4_FMT_Q8_0) return gemm::launch_fmt<gemm::GemmQ8_0>(w, x, y, m, k, n, s, cus);
    if (fmt == Q4_FMT_Q2_K) return gemm::launch_fmt<gemm::GemmQ2_K>(w, x, y, m, k, n, s, cus);
    if (fmt == Q4_FMT_Q1_0) return gemm::launch_fmt<gemm::GemmQ1_0>(w, x, y, m, k, n, s, cus);
    return gemm::launch_fmt<gemm::GemmQ4_K>(w, x, y, m, k, n, s, cus);
}

}  // namespace q4

extern "C" int q4_gemm_tuned(int fmt, const void *w, const uint16_t *x_bf16, float *y, int64_t m, int64_t k,
                             int64_t n, const q4_gemm_tuning *tuning, void *hip_stream)
{
    const int st = q4::check_product_args(fmt, w, x_bf16, y, m, k, n, INT64_MAX);
    if (st != Q4_OK) return st;
    if (!tuning || tuning->tile_rows < 0 || tuning->tile_tokens < 0 || tuning->stage_k < 0) return Q4_EINVAL;
    if (m == 0 || n == 0) return Q4_OK;
    if (n >= (1LL << 22)) return Q4_EUNSUPPORTED;
    const int tm = tuning->tile_rows ? tuning->tile_rows : 32;
    const int tn = tuning->tile_tokens ? tuning->tile_tokens : 64;
    const int kc = tuning->stage_k ? tuning->stage_k : 256;
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    if (fmt == Q4_FMT_Q4_0) return q4::gemm::launch_geometry<q4::gemm::GemmQ4_0>(tm, tn, kc, w, x_bf16, y, m, k, n, s);
    if (fmt == Q4_FMT_Q8_0) return q4::gemm::launch_geometry<q4::gemm::GemmQ8_0>(tm, tn, kc, w, x_bf16, y, m, k, n, s);
    if (fmt == Q4_FMT_Q2_K) return q4::gemm::launch_geometry<q4::gemm::GemmQ2_K>(tm, tn, kc, w, x_bf16, y, m, k, n, s);
    if (fmt == Q4_FMT_Q1_0) return q4::gemm::launch_geometry<q4::gemm::GemmQ1_0>(tm, tn, kc, w, x_bf16, y, m, k, n, s);
    return q4::gemm::launch_geometry<q4::gemm::GemmQ4_K>(tm, tn, kc, w, x_bf16, y, m, k, n, s);
}

extern "C" int q4_gemm(int fmt, const void *w, const uint16_t *x_bf16, float *y, int64_t m, int64_t k, int64_t n,
                       void *hip_stream)
{
    const int st = q4::check_product_args(fmt, w, x_bf16, y, m, k, n, INT64_MAX);
    if (st != Q4_OK) return st;
    if (m == 0 || n == 0) return Q4_OK;
    if (n >= (1LL << 22)) return Q4_EUNSUPPORTED;
    return q4::launch_gemm(fmt, w, x_bf16, y, m, k, n, hip_stream);
}
