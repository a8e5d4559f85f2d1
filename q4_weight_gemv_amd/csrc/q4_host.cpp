// Host part of the library: buffer sizes, status strings and the reference
// quantizer that produces the weight buffers the device products read.
//
// Quantization is the offline step that turns 16/32-bit weights into 4 bits
// per parameter (MicroLLM Lab post, "Seven models, all in Q4"); the device
// products never quantize. Rounding to fp16 uses the compiler's _Float16
// conversion (IEEE round-to-nearest-even); codes round half away from zero.
//
// Compiled with -ffp-contract=off: every expression rounds as written, so the
// buffers are a deterministic function of the input floats.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>

#include "q4.h"

namespace {

inline uint16_t half_bits(_Float16 h)
{
    uint16_t b;
    std::memcpy(&b, &h, 2);
    return b;
}

inline bool half_is_finite(_Float16 h) { return (half_bits(h) & 0x7C00u) != 0x7C00u; }

// round_half_away(v) + bias, clamped to [0, hi].
inline int code_of(double v, int bias, int hi)
{
    double r = std::round(v) + bias;  // std::round: half away from zero
    if (r < 0.0) return 0;
    if (r > hi) return hi;
    return static_cast<int>(r);
}

// ---- Q4_0 -----------------------------------------------------------------

// Quantize row r of a Q4_0 matrix into the two planes. Returns the status and,
// on failure, the failing block's index within the row.
int q4_0_row(const float *wr, int64_t nb, uint8_t *nib_row, uint8_t *scale_row, int64_t *bad)
{
    for (int64_t b = 0; b < nb; b++) {
        const float *v = wr + 32 * b;
        float amax = 0.0f;
        bool finite = true;
        for (int i = 0; i < 32; i++) {
            finite = finite && std::isfinite(v[i]);
            amax = std::max(amax, std::fabs(v[i]));
        }
        if (!finite) { *bad = b; return Q4_ENONFINITE; }
        _Float16 dh = static_cast<_Float16>(amax / 7.0f);
        if (!half_is_finite(dh)) { *bad = b; return Q4_ERANGE; }
        const double d = static_cast<double>(static_cast<float>(dh));
        uint8_t codes[32];
        for (int i = 0; i < 32; i++)
            codes[i] = d == 0.0 ? 8 : static_cast<uint8_t>(code_of(v[i] / d, 8, 15));
        for (int j = 0; j < 16; j++) nib_row[16 * b + j] = static_cast<uint8_t>(codes[j] | (codes[16 + j] << 4));
        const uint16_t bits = half_bits(dh);
        scale_row[2 * b] = static_cast<uint8_t>(bits);
        scale_row[2 * b + 1] = static_cast<uint8_t>(bits >> 8);
    }
    return Q4_OK;
}

// ---- Q8_0 -----------------------------------------------------------------

// Quantize row r of a Q8_0 matrix into the code and scale planes.
int q8_0_row(const float *wr, int64_t nb, uint8_t *code_row, uint8_t *scale_row, int64_t *bad)
{
    for (int64_t b = 0; b < nb; b++) {
        const float *v = wr + 32 * b;
        float amax = 0.0f;
        bool finite = true;
        for (int i = 0; i < 32; i++) {
            finite = finite && std::isfinite(v[i]);
            amax = std::max(amax, std::fabs(v[i]));
        }
        if (!finite) { *bad = b; return Q4_ENONFINITE; }
        _Float16 dh = static_cast<_Float16>(amax / 127.0f);
        if (!half_is_finite(dh)) { *bad = b; return Q4_ERANGE; }
        const double d = static_cast<double>(static_cast<float>(dh));
        for (int i = 0; i < 32; i++) {
            // code_of clamps to [0, 254] around the bias 127: codes -127..127.
            const int q = d == 0.0 ? 0 : code_of(v[i] / d, 127, 254) - 127;
            code_row[32 * b + i] = static_cast<uint8_t>(static_cast<int8_t>(q));
        }
        const uint16_t bits = half_bits(dh);
        scale_row[2 * b] = static_cast<uint8_t>(bits);
        scale_row[2 * b + 1] = static_cast<uint8_t>(bits >> 8);
    }
    return Q4_OK;
}

// ---- Q1_0 -----------------------------------------------------------------

// Quantize row r of a Q1_0 matrix into the bit and scale planes.
int q1_0_row(const float *wr, int64_t nb, uint8_t *bit_row, uint8_t *scale_row, int64_t *bad)
{
    for (int64_t b = 0; b < nb; b++) {
        const float *v = wr + 32 * b;
        double total = 0.0;
        bool finite = true;
        uint32_t word = 0;
        for (int i = 0; i < 32; i++) {
            finite = finite && std::isfinite(v[i]);
            total += std::fabs(static_cast<double>(v[i]));
            if (!(v[i] < 0.0f)) word |= 1u << i;
        }
        if (!finite) { *bad = b; return Q4_ENONFINITE; }
        // One rounding, float64 -> fp16 (round to nearest even).
        _Float16 dh = static_cast<_Float16>(total / 32.0);
        if (!half_is_finite(dh)) { *bad = b; return Q4_ERANGE; }
        for (int j = 0; j < 4; j++) bit_row[4 * b + j] = static_cast<uint8_t>(word >> (8 * j));
        const uint16_t bits = half_bits(dh);
        scale_row[2 * b] = static_cast<uint8_t>(bits);
        scale_row[2 * b + 1] = static_cast<uint8_t>(bits >> 8);
    }
    return Q4_OK;
}

// ---- Q4_K -----------------------------------------------------------------

inline void pack_6bit(const uint8_t sc[8], const uint8_t mn[8], uint8_t S[12])
{
    // Sub-blocks 0..3 keep their 6 bits in S[0..7]; sub-blocks 4..7 put their
    // low 4 bits in S[8..11] and their top 2 bits in the top of S[0..7].
    for (int j = 0; j < 4; j++) {
        S[j] = static_cast<uint8_t>((sc[j] & 63) | ((sc[j + 4] >> 4) << 6));
        S[j + 4] = static_cast<uint8_t>((mn[j] & 63) | ((mn[j + 4] >> 4) << 6));
        S[j + 8] = static_cast<uint8_t>((sc[j + 4] & 15) | ((mn[j + 4] & 15) << 4));
    }
}

int q4_k_superblock(const float *v, uint8_t *out)
{
    double step[8], off[8];
    double smax = 0.0, mumax = 0.0;
    for (int i = 0; i < 256; i++)
        if (!std::isfinite(v[i])) return Q4_ENONFINITE;
    for (int j = 0; j < 8; j++) {
        const float *s = v + 32 * j;
        double mn = std::min(0.0, static_cast<double>(*std::min_element(s, s + 32)));
        double mx = static_cast<double>(*std::max_element(s, s + 32));
        step[j] = (mx - mn) / 15.0;
        off[j] = -mn;
        smax = std::max(smax, step[j]);
        mumax = std::max(mumax, off[j]);
    }
    _Float16 dh = static_cast<_Float16>(smax / 63.0);
    _Float16 mh = static_cast<_Float16>(mumax / 63.0);
    if (!half_is_finite(dh) || !half_is_finite(mh)) return Q4_ERANGE;
    const double d = static_cast<float>(dh);
    const double dmin = static_cast<float>(mh);
    uint8_t sc[8], mn[8];
    for (int j = 0; j < 8; j++) {
        sc[j] = d == 0.0 ? 0 : static_cast<uint8_t>(code_of(step[j] / d, 0, 63));
        mn[j] = dmin == 0.0 ? 0 : static_cast<uint8_t>(code_of(off[j] / dmin, 0, 63));
    }
    uint8_t q[256];
    for (int j = 0; j < 8; j++) {
        const double st = d * sc[j];
        const double o = dmin * mn[j];
        for (int i = 0; i < 32; i++)
            q[32 * j + i] = st == 0.0 ? 0 : static_cast<uint8_t>(code_of((v[32 * j + i] + o) / st, 0, 15));
    }
    const uint16_t db = half_bits(dh), mb = half_bits(mh);
    out[0] = static_cast<uint8_t>(db);
    out[1] = static_cast<uint8_t>(db >> 8);
    out[2] = static_cast<uint8_t>(mb);
    out[3] = static_cast<uint8_t>(mb >> 8);
    pack_6bit(sc, mn, out + 4);
    for (int c = 0; c < 4; c++)
        for (int i = 0; i < 32; i++)
            out[16 + 32 * c + i] = static_cast<uint8_t>(q[64 * c + i] | (q[64 * c + 32 + i] << 4));
    return Q4_OK;
}

// ---- Q2_K -----------------------------------------------------------------

// One 256-weight super-block into its three fields: 64 code bytes, 16 scale
// bytes (sc | mn << 4 per 16-weight sub-block) and fp16 d, dmin.
int q2_k_superblock(const float *v, uint8_t *codes, uint8_t *scales, uint8_t *dd)
{
    double step[16], off[16];
    double smax = 0.0, mumax = 0.0;
    for (int i = 0; i < 256; i++)
        if (!std::isfinite(v[i])) return Q4_ENONFINITE;
    for (int j = 0; j < 16; j++) {
        const float *s = v + 16 * j;
        double mn = std::min(0.0, static_cast<double>(*std::min_element(s, s + 16)));
        double mx = static_cast<double>(*std::max_element(s, s + 16));
        step[j] = (mx - mn) / 3.0;
        off[j] = -mn;
        smax = std::max(smax, step[j]);
        mumax = std::max(mumax, off[j]);
    }
    _Float16 dh = static_cast<_Float16>(smax / 15.0);
    _Float16 mh = static_cast<_Float16>(mumax / 15.0);
    if (!half_is_finite(dh) || !half_is_finite(mh)) return Q4_ERANGE;
    const double d = static_cast<float>(dh);
    const double dmin = static_cast<float>(mh);
    int sc[16], mn[16];
    for (int j = 0; j < 16; j++) {
        sc[j] = d == 0.0 ? 0 : code_of(step[j] / d, 0, 15);
        mn[j] = dmin == 0.0 ? 0 : code_of(off[j] / dmin, 0, 15);
        scales[j] = static_cast<uint8_t>(sc[j] | (mn[j] << 4));
    }
    std::memset(codes, 0, 64);
    for (int h = 0; h < 2; h++)
        for (int j = 0; j < 4; j++)
            for (int r = 0; r < 32; r++) {
                const int e = 128 * h + 32 * j + r;
                const double st = d * sc[e / 16];
                const double o = dmin * mn[e / 16];
                const int q = st == 0.0 ? 0 : code_of((v[e] + o) / st, 0, 3);
                codes[32 * h + r] = static_cast<uint8_t>(codes[32 * h + r] | (q << (2 * j)));
            }
    const uint16_t db = half_bits(dh), mb = half_bits(mh);
    dd[0] = static_cast<uint8_t>(db);
    dd[1] = static_cast<uint8_t>(db >> 8);
    dd[2] = static_cast<uint8_t>(mb);
    dd[3] = static_cast<uint8_t>(mb >> 8);
    return Q4_OK;
}

// Run fn(row, &bad_col_block) over rows on a few threads; return the status
// of the first failing block in row-major order.
template <class F>
int for_rows(int64_t m, int64_t blocks_per_row, F fn)
{
    const int64_t total = m * blocks_per_row;
    unsigned hw = std::max(1u, std::thread::hardware_concurrency());
    int nth = static_cast<int>(std::min<int64_t>(std::min<unsigned>(hw, 16u), std::max<int64_t>(1, total / 4096)));
    if (nth <= 1) {
        for (int64_t r = 0; r < m; r++) {
            int64_t bad = 0;
            int st = fn(r, &bad);
            if (st != Q4_OK) return st;
        }
        return Q4_OK;
    }
    std::vector<int64_t> first(nth, INT64_MAX);
    std::vector<int> status(nth, Q4_OK);
    std::vector<std::thread> th;
    const int64_t per = (m + nth - 1) / nth;
    for (int t = 0; t < nth; t++) {
        th.emplace_back([&, t] {
            for (int64_t r = t * per; r < std::min(m, (t + 1) * per); r++) {
                int64_t bad = 0;
                int st = fn(r, &bad);
                if (st != Q4_OK) {
                    first[t] = r * blocks_per_row + bad;
                    status[t] = st;
                    return;
                }
            }
        });
    }
    for (auto &x : th) x.join();
    int64_t best = INT64_MAX;
    int st = Q4_OK;
    for (int t = 0; t < nth; t++)
        if (first[t] < best) { best = first[t]; st = status[t]; }
    return st;
}

}  // namespace

extern "C" {

size_t q4_weight_bytes(int fmt, int64_t m, int64_t k)
{
    if (m < 0 || k <= 0) return 0;
    if (fmt == Q4_FMT_Q4_0) return k % 32 ? 0 : static_cast<size_t>(m) * static_cast<size_t>(k / 32) * 18u;
    if (fmt == Q4_FMT_Q4_K) return k % 256 ? 0 : static_cast<size_t>(m) * static_cast<size_t>(k / 256) * 144u;
    if (fmt == Q4_FMT_Q8_0) return k % 32 ? 0 : static_cast<size_t>(m) * static_cast<size_t>(k / 32) * 34u;
    if (fmt == Q4_FMT_Q2_K) return k % 256 ? 0 : static_cast<size_t>(m) * static_cast<size_t>(k / 256) * 84u;
    if (fmt == Q4_FMT_Q1_0) return k % 32 ? 0 : static_cast<size_t>(m) * static_cast<size_t>(k / 32) * 6u;
    return 0;
}

int q4_quantize_ref(int fmt, const float *w, int64_t m, int64_t k, void *out, size_t out_bytes)
{
    if (fmt != Q4_FMT_Q4_0 && fmt != Q4_FMT_Q4_K && fmt != Q4_FMT_Q8_0 && fmt != Q4_FMT_Q2_K && fmt != Q4_FMT_Q1_0)
        return Q4_EUNSUPPORTED;
    const size_t need = q4_weight_bytes(fmt, m, k);
    const int64_t blk = fmt == Q4_FMT_Q4_K || fmt == Q4_FMT_Q2_K ? 256 : 32;
    if (need == 0 && !(m == 0 && k > 0 && k % blk == 0)) return Q4_EINVAL;
    if (m == 0) return Q4_OK;
    if (!w || !out || out_bytes < need) return Q4_EINVAL;
    uint8_t *o = static_cast<uint8_t *>(out);
    if (fmt == Q4_FMT_Q4_0) {
        const int64_t nb = k / 32;
        uint8_t *nib = o;
        uint8_t *scl = o + static_cast<size_t>(m) * static_cast<size_t>(k) / 2;
        return for_rows(m, nb, [&](int64_t r, int64_t *bad) {
            return q4_0_row(w + r * k, nb, nib + r * nb * 16, scl + r * nb * 2, bad);
        });
    }
    if (fmt == Q4_FMT_Q8_0) {
        const int64_t nb = k / 32;
        uint8_t *codes = o;
        uint8_t *scl = o + static_cast<size_t>(m) * static_cast<size_t>(k);
        return for_rows(m, nb, [&](int64_t r, int64_t *bad) {
            return q8_0_row(w + r * k, nb, codes + r * nb * 32, scl + r * nb * 2, bad);
        });
    }
    if (fmt == Q4_FMT_Q1_0) {
        const int64_t nb = k / 32;
        uint8_t *bits = o;
        uint8_t *scl = o + static_cast<size_t>(m) * static_cast<size_t>(k) / 8;
        return for_rows(m, nb, [&](int64_t r, int64_t *bad) {
            return q1_0_row(w + r * k, nb, bits + r * nb * 4, scl + r * nb * 2, bad);
        });
    }
    const int64_t ns = k / 256;
    if (fmt == Q4_FMT_Q2_K) {
        uint8_t *scl = o + static_cast<size_t>(m) * static_cast<size_t>(k) / 4;
        uint8_t *dd = scl + static_cast<size_t>(m) * static_cast<size_t>(k) / 16;
        return for_rows(m, ns, [&](int64_t r, int64_t *bad) {
            for (int64_t s = 0; s < ns; s++) {
                const int64_t i = r * ns + s;
                int st = q2_k_superblock(w + r * k + s * 256, o + i * 64, scl + i * 16, dd + i * 4);
                if (st != Q4_OK) { *bad = s; return st; }
            }
            return static_cast<int>(Q4_OK);
        });
    }
    return for_rows(m, ns, [&](int64_t r, int64_t *bad) {
        for (int64_t s = 0; s < ns; s++) {
            int st = q4_k_superblock(w + r * k + s * 256, o + (r * ns + s) * 144);
            if (st != Q4_OK) { *bad = s; return st; }
        }
        return static_cast<int>(Q4_OK);
    });
}

const char *q4_strerror(int status)
{
    switch (status) {
    case Q4_OK: return "ok";
    case Q4_EINVAL: return "invalid argument (size, null pointer, block multiple or buffer length)";
    case Q4_EUNSUPPORTED: return "unsupported (format, token count, or size beyond 32-bit offsets)";
    case Q4_EALIGN: return "misaligned pointer (w needs 16 bytes, activations and outputs 4, norm vectors and caches 16)";
    case Q4_ENONFINITE: return "non-finite weight given to the quantizer";
    case Q4_ERANGE: return "block scale overflows fp16";
    case Q4_EHIP: return "HIP runtime error";
    default: return "unknown status";
    }
}

}  // extern "C"
