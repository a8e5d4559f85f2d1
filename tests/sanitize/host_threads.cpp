// Thread check of the host quantizer (q4_quantize_ref), built with a thread
// sanitizer by tests/sanitize/run.py: every format on matrices large enough
// that the quantizer splits the rows over several threads, against the same
// rows quantized one call per row (one thread), byte for byte; and the status
// of a matrix with failing blocks in several threads' row ranges, which must
// be that of the first failing block in row-major order.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <random>
#include <vector>

#include "q4.h"

static int check_format(int fmt, int64_t m, int64_t k, std::mt19937_64 &rng)
{
    std::normal_distribution<float> nd(0.0f, 0.02f);
    std::vector<float> w(static_cast<size_t>(m * k));
    for (auto &v : w) v = nd(rng);
    const size_t bytes = q4_weight_bytes(fmt, m, k);
    std::vector<uint8_t> whole(bytes), rows(bytes);
    if (q4_quantize_ref(fmt, w.data(), m, k, whole.data(), bytes) != Q4_OK) return 1;
    // Row by row: each row alone is a one-row matrix with its own planes;
    // re-place its planes at the row's offsets of the whole matrix.
    const size_t per_row = q4_weight_bytes(fmt, 1, k);
    std::vector<uint8_t> one(per_row);
    // Plane sizes per row, in the order the layouts place them (header q4.h).
    std::vector<size_t> planes;
    if (fmt == Q4_FMT_Q4_0) planes = {static_cast<size_t>(k / 2), static_cast<size_t>(k / 16)};
    else if (fmt == Q4_FMT_Q8_0) planes = {static_cast<size_t>(k), static_cast<size_t>(k / 16)};
    else if (fmt == Q4_FMT_Q1_0) planes = {static_cast<size_t>(k / 8), static_cast<size_t>(k / 16)};
    else if (fmt == Q4_FMT_Q2_K) planes = {static_cast<size_t>(k / 4), static_cast<size_t>(k / 16), static_cast<size_t>(k / 64)};
    else planes = {per_row};  // Q4_K: row-major super-blocks, one plane
    for (int64_t r = 0; r < m; r++) {
        if (q4_quantize_ref(fmt, w.data() + r * k, 1, k, one.data(), per_row) != Q4_OK) return 2;
        size_t src = 0, base = 0;
        for (size_t p : planes) {
            std::memcpy(rows.data() + base + static_cast<size_t>(r) * p, one.data() + src, p);
            src += p;
            base += p * static_cast<size_t>(m);
        }
    }
    if (whole != rows) return 3;
    // Failing blocks in the last thread's rows and, later in row-major order
    // than an earlier failure, in the first thread's rows.
    w[static_cast<size_t>((m - 1) * k + 5)] = NAN;
    w[static_cast<size_t>(3 * k + 40)] = INFINITY;
    w[static_cast<size_t>(7 * k + 1)] = 1e30f;
    if (q4_quantize_ref(fmt, w.data(), m, k, whole.data(), bytes) != Q4_ENONFINITE) return 4;
    return 0;
}

int main()
{
    std::mt19937_64 rng(2024);
    const int fmts[] = {Q4_FMT_Q4_0, Q4_FMT_Q4_K, Q4_FMT_Q8_0, Q4_FMT_Q2_K, Q4_FMT_Q1_0};
    for (int fmt : fmts) {
        const int st = check_format(fmt, 512, 4096, rng);
        std::printf("format %d: %s\n", fmt, st == 0 ? "ok" : "FAILED");
        if (st) return st;
    }
    return 0;
}
