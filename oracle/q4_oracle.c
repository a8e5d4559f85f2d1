/*
 * q4_oracle.c -- plain, slow, obviously-correct CPU reference for the Q4
 * weight matrix products.  TEST INFRASTRUCTURE ONLY: the tests, the smoke
 * check and the bench's CPU-baseline leg load it; the product library never
 * does, and the two share no source, header, table or helper.
 *
 * What it computes, and where that is defined:
 *   - Weights are stored block-quantized to 4 bits and dequantized inside
 *     the matrix products: in registers for the decode matrix-vector
 *     product, through shared memory for the prefill matrix-matrix product
 *     (Llamas on the Web, technical summary, Methodology section 3,
 *     "integrated dequantization").
 *   - Formats are flat byte buffers whose decoding is a per-format routine
 *     (same section, "extensibility"); 16-bit weights become 4 bits per
 *     parameter (MicroLLM Lab post, "Seven models, all in Q4").
 *   - Q4_0 (llama.cpp's legacy 4-bit scheme, one of the "legacy" formats the
 *     technical summary's problem statement lists): blocks of 32 weights, an
 *     fp16 scale d = max|w| / 7, codes q in [0, 15], value (q - 8) * d.
 *   - Q4_K (the K-quant family named by q4_k_m in the summary's results):
 *     256-weight super-blocks of eight 32-weight sub-blocks, each with a 6-bit
 *     scale and a 6-bit min, plus fp16 d and dmin; value d*sc*q - dmin*m.
 *   - Q2_K (the summary's q2_k): 256-weight super-blocks of sixteen 16-weight
 *     sub-blocks with 4-bit scales and mins, fp16 d and dmin, 2-bit codes;
 *     value d*sc*q - dmin*m.
 *   - Q8_0 (the q8_0 the summary's results compare with q4_k_m and q2_k):
 *     blocks of 32 weights, an fp16 scale d = max|w| / 127, codes q in
 *     [-127, 127] stored as bytes, value q * d.
 *   - Q1_0 (the 1-bit format the technical summary names as an example of a
 *     format added by writing one dequantization routine): blocks of 32
 *     weights, an fp16 scale d = mean |w|, one sign bit per weight, value
 *     +d or -d.
 *   - The gated product silu(g) * u of a stacked gate/up matrix (kernel
 *     fusion: WebGPT README, "Roadmap"; the summary's experimental results).
 *
 * The pages give no bit layout, tie rule or quantizer search; the readings
 * used here (plane-split Q4_0 buffer, llama.cpp nibble order, half-away-from-
 * zero rounding, the min/max Q4_K quantizer) are listed with their reasons in
 * the design notes at the repository root.
 *
 * Build: gcc -std=c99 -O2 -ffp-contract=off -fno-fast-math (no contraction, so
 * every float expression below rounds exactly as written).
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_EINVAL (-1)
#define ORACLE_ENONFINITE (-4)
#define ORACLE_ERANGE (-5)

/* ------------------------------------------------------------------------
 * IEEE-754 binary16 and bfloat16, written from the format definitions.
 * A finite binary16 value is (-1)^s * 2^(E-15) * (1 + f/1024) for
 * 1 <= E <= 30 and (-1)^s * 2^-14 * (f/1024) for E = 0.
 * ------------------------------------------------------------------------ */

float oracle_fp16_to_fp32(uint16_t h)
{
    int s = (h >> 15) & 1;
    int e = (h >> 10) & 0x1F;
    int f = h & 0x3FF;
    double v;
    if (e == 0x1F) {
        if (f != 0) return NAN;
        return s ? -INFINITY : INFINITY;
    }
    if (e == 0)
        v = ldexp((double)f, -24);               /* 2^-14 * f / 2^10 */
    else
        v = ldexp((double)(1024 + f), e - 25);   /* 2^(e-15) * (1024+f) / 2^10 */
    return (float)(s ? -v : v);                  /* exact: <= 11 significant bits */
}

/* Round a double (finite, or not) to the nearest binary16, ties to even. */
uint16_t oracle_f64_to_fp16(double v)
{
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (isnan(v)) return (uint16_t)(sign | 0x7E00);
    if (isinf(v)) return (uint16_t)(sign | 0x7C00);
    if (a == 0.0) return sign;
    /* Exponent of the binade holding a, never below the subnormal binade. */
    int ex;
    frexp(a, &ex);                 /* a = m * 2^ex, m in [0.5, 1) -> binade 2^(ex-1) */
    int E = ex - 1;
    if (E < -14) E = -14;
    /* Spacing of binary16 values in that binade: 2^(E-10). */
    double n = ldexp(a, 10 - E);   /* exact: scaling by a power of two */
    double nf = floor(n);
    double frac = n - nf;          /* exact */
    if (frac > 0.5 || (frac == 0.5 && fmod(nf, 2.0) != 0.0)) nf += 1.0;
    /* nf * 2^(E-10) is the rounded magnitude; nf may have carried to 2048. */
    if (nf >= 2048.0) { nf /= 2.0; E += 1; }
    if (E > 15) return (uint16_t)(sign | 0x7C00);           /* overflow */
    if (nf < 1024.0) return (uint16_t)(sign | (uint16_t)nf); /* subnormal (E == -14) */
    return (uint16_t)(sign | (uint16_t)((E + 15) << 10) | (uint16_t)(nf - 1024.0));
}

uint16_t oracle_fp32_to_fp16(float f) { return oracle_f64_to_fp16((double)f); }

/* bfloat16 is the top half of binary32; rounding keeps 8 significant bits. */
float oracle_bf16_to_fp32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

uint16_t oracle_fp32_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    if (isnan(f)) return (uint16_t)((u >> 16) | 0x40);
    if (isinf(f) || f == 0.0f) return (uint16_t)(u >> 16);
    /* Value in units of the bf16 spacing of f's binade: round that to an
     * integer with ties to even, then rebuild. Done in double (exact). */
    double a = fabs((double)f);
    int ex;
    frexp(a, &ex);
    int E = ex - 1;
    if (E < -126) E = -126;                 /* binary32 subnormal binade */
    double n = ldexp(a, 7 - E);             /* spacing 2^(E-7) */
    double nf = floor(n);
    double frac = n - nf;
    if (frac > 0.5 || (frac == 0.5 && fmod(nf, 2.0) != 0.0)) nf += 1.0;
    double r = ldexp(nf, E - 7);
    float rf = (float)r;                    /* exact, or +inf on overflow */
    if (signbit(f)) rf = -rf;
    uint32_t ru;
    memcpy(&ru, &rf, 4);
    return (uint16_t)(ru >> 16);
}

/* Round half away from zero (C's round()), used for every code in both formats. */
static double round_half_away(double v) { return round(v); }

static int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

/* ------------------------------------------------------------------------
 * Q4_0.  Buffer for an m x k matrix (k a multiple of 32), "plane-split":
 *   bytes [0, m*k/2)          nibble plane: block (r, b) at (r*k/32 + b)*16,
 *                             byte j: low nibble = element j, high nibble =
 *                             element j + 16 of the block (llama.cpp order);
 *   bytes [m*k/2, m*k*9/16)   scale plane: fp16 d of block (r, b) at
 *                             m*k/2 + (r*k/32 + b)*2, little-endian.
 * ------------------------------------------------------------------------ */

size_t oracle_q4_0_bytes(int64_t m, int64_t k) { return (size_t)(m * k / 32) * 18u; }

/* One block: 32 floats -> 16 nibble bytes and the fp16 scale bits. */
int oracle_q4_0_quantize_block(const float *w, uint8_t *nib, uint16_t *d_bits)
{
    float amax = 0.0f;
    for (int i = 0; i < 32; i++) {
        if (!isfinite(w[i])) return ORACLE_ENONFINITE;
        float a = fabsf(w[i]);
        if (a > amax) amax = a;
    }
    float d32 = amax / 7.0f;                          /* binary32 division */
    uint16_t dh = oracle_fp32_to_fp16(d32);
    if ((dh & 0x7C00) == 0x7C00) return ORACLE_ERANGE; /* scale not finite in fp16 */
    float d = oracle_fp16_to_fp32(dh);
    int q[32];
    for (int i = 0; i < 32; i++) {
        if (d == 0.0f) {
            q[i] = 8;
        } else {
            /* exact quotient up to double rounding, which cannot create or
             * remove a tie: both operands carry at most 24 significant bits */
            double t = (double)w[i] / (double)d;
            q[i] = clampi((int)round_half_away(t) + 8, 0, 15);
        }
    }
    for (int j = 0; j < 16; j++) nib[j] = (uint8_t)(q[j] | (q[j + 16] << 4));
    *d_bits = dh;
    return ORACLE_OK;
}

int oracle_q4_0_quantize(const float *w, int64_t m, int64_t k, uint8_t *out)
{
    if (m < 0 || k <= 0 || k % 32 != 0) return ORACLE_EINVAL;
    int64_t nb = k / 32;
    uint8_t *nibs = out;
    uint8_t *scales = out + (size_t)(m * k / 2);
    for (int64_t r = 0; r < m; r++) {
        for (int64_t b = 0; b < nb; b++) {
            uint16_t dh;
            int st = oracle_q4_0_quantize_block(w + r * k + b * 32, nibs + (r * nb + b) * 16, &dh);
            if (st != ORACLE_OK) return st;
            scales[(r * nb + b) * 2] = (uint8_t)(dh & 0xFF);
            scales[(r * nb + b) * 2 + 1] = (uint8_t)(dh >> 8);
        }
    }
    return ORACLE_OK;
}

/* Dequantized weight (r, c): (q - 8) * d, exact in binary32. */
float oracle_q4_0_weight(const uint8_t *buf, int64_t m, int64_t k, int64_t r, int64_t c)
{
    int64_t nb = k / 32;
    int64_t b = c / 32;
    int64_t e = c % 32;
    const uint8_t *blk = buf + (r * nb + b) * 16;
    int q = (e < 16) ? (blk[e] & 0x0F) : (blk[e - 16] >> 4);
    const uint8_t *s = buf + (size_t)(m * k / 2) + (r * nb + b) * 2;
    uint16_t dh = (uint16_t)(s[0] | (s[1] << 8));
    float d = oracle_fp16_to_fp32(dh);
    return (float)(q - 8) * d;
}

void oracle_q4_0_dequantize(const uint8_t *buf, int64_t m, int64_t k, float *w_hat)
{
    for (int64_t r = 0; r < m; r++)
        for (int64_t c = 0; c < k; c++)
            w_hat[r * k + c] = oracle_q4_0_weight(buf, m, k, r, c);
}

/* llama.cpp's array-of-blocks form (per block: fp16 d, then 16 nibble bytes)
 * to and from the plane-split form; a bijection that moves no bits. */
void oracle_q4_0_planes_to_aos(const uint8_t *planes, int64_t m, int64_t k, uint8_t *aos)
{
    int64_t nblk = m * k / 32;
    const uint8_t *scales = planes + (size_t)(m * k / 2);
    for (int64_t i = 0; i < nblk; i++) {
        aos[i * 18] = scales[i * 2];
        aos[i * 18 + 1] = scales[i * 2 + 1];
        memcpy(aos + i * 18 + 2, planes + i * 16, 16);
    }
}

void oracle_q4_0_aos_to_planes(const uint8_t *aos, int64_t m, int64_t k, uint8_t *planes)
{
    int64_t nblk = m * k / 32;
    uint8_t *scales = planes + (size_t)(m * k / 2);
    for (int64_t i = 0; i < nblk; i++) {
        scales[i * 2] = aos[i * 18];
        scales[i * 2 + 1] = aos[i * 18 + 1];
        memcpy(planes + i * 16, aos + i * 18 + 2, 16);
    }
}

/* ------------------------------------------------------------------------
 * Q8_0 (llama.cpp's legacy 8-bit scheme, the q8_0 that the technical
 * summary's results compare with q4_k_m and q2_k): blocks of 32 weights, an
 * fp16 scale d = max|w| / 127, codes q in [-127, 127], value q * d.
 * Buffer for an m x k matrix, plane-split like Q4_0:
 *   bytes [0, m*k)            code plane: block (r, b) at (r*k/32 + b)*32,
 *                             byte j = code of element j (two's complement);
 *   bytes [m*k, m*k*17/16)    scale plane: fp16 d of block (r, b) at
 *                             m*k + (r*k/32 + b)*2, little-endian.
 * ------------------------------------------------------------------------ */

size_t oracle_q8_0_bytes(int64_t m, int64_t k) { return (size_t)(m * k / 32) * 34u; }

/* One block: 32 floats -> 32 codes and the fp16 scale bits. */
int oracle_q8_0_quantize_block(const float *w, int8_t *q, uint16_t *d_bits)
{
    float amax = 0.0f;
    for (int i = 0; i < 32; i++) {
        if (!isfinite(w[i])) return ORACLE_ENONFINITE;
        float a = fabsf(w[i]);
        if (a > amax) amax = a;
    }
    float d32 = amax / 127.0f;                        /* binary32 division */
    uint16_t dh = oracle_fp32_to_fp16(d32);
    if ((dh & 0x7C00) == 0x7C00) return ORACLE_ERANGE; /* scale not finite in fp16 */
    float d = oracle_fp16_to_fp32(dh);
    for (int i = 0; i < 32; i++) {
        if (d == 0.0f) {
            q[i] = 0;
        } else {
            /* exact quotient up to double rounding (see the Q4_0 block) */
            double t = (double)w[i] / (double)d;
            q[i] = (int8_t)clampi((int)round_half_away(t), -127, 127);
        }
    }
    *d_bits = dh;
    return ORACLE_OK;
}

int oracle_q8_0_quantize(const float *w, int64_t m, int64_t k, uint8_t *out)
{
    if (m < 0 || k <= 0 || k % 32 != 0) return ORACLE_EINVAL;
    int64_t nb = k / 32;
    uint8_t *scales = out + (size_t)(m * k);
    for (int64_t r = 0; r < m; r++) {
        for (int64_t b = 0; b < nb; b++) {
            uint16_t dh;
            int8_t q[32];
            int st = oracle_q8_0_quantize_block(w + r * k + b * 32, q, &dh);
            if (st != ORACLE_OK) return st;
            memcpy(out + (r * nb + b) * 32, q, 32);
            scales[(r * nb + b) * 2] = (uint8_t)(dh & 0xFF);
            scales[(r * nb + b) * 2 + 1] = (uint8_t)(dh >> 8);
        }
    }
    return ORACLE_OK;
}

/* Dequantized weight (r, c): q * d, exact in binary32 (8 + 11 significant bits). */
float oracle_q8_0_weight(const uint8_t *buf, int64_t m, int64_t k, int64_t r, int64_t c)
{
    int64_t nb = k / 32;
    int64_t b = c / 32;
    int q = (int)(int8_t)buf[(r * nb + b) * 32 + c % 32];
    const uint8_t *s = buf + (size_t)(m * k) + (r * nb + b) * 2;
    float d = oracle_fp16_to_fp32((uint16_t)(s[0] | (s[1] << 8)));
    return (float)q * d;
}

void oracle_q8_0_dequantize(const uint8_t *buf, int64_t m, int64_t k, float *w_hat)
{
    for (int64_t r = 0; r < m; r++)
        for (int64_t c = 0; c < k; c++)
            w_hat[r * k + c] = oracle_q8_0_weight(buf, m, k, r, c);
}

/* ------------------------------------------------------------------------
 * Q1_0 (the 1-bit format the technical summary's extensibility point names;
 * the pages define no more than that it holds 1-bit models). Reading: the
 * Q4_0 block structure with a one-bit code. Blocks of 32 weights; code
 * b = 1 for w >= 0 (either zero included), 0 for w < 0; one fp16 scale
 * d = RNE(sum |w| / 32) (float64 sum and quotient), the least-squares scale
 * for codes of fixed sign: sum (w - d s)^2 with s = +-1 is smallest at
 * d = mean |w|. Value (2b - 1) * d, exact in binary32.
 * Buffer for an m x k matrix, plane-split like Q4_0:
 *   bytes [0, m*k/8)          bit plane: block (r, b) at (r*k/32 + b)*4, a
 *                             little-endian 32-bit word whose bit e is the
 *                             code of element e;
 *   bytes [m*k/8, m*k*3/16)   scale plane: fp16 d of block (r, b) at
 *                             m*k/8 + (r*k/32 + b)*2, little-endian.
 * ------------------------------------------------------------------------ */

size_t oracle_q1_0_bytes(int64_t m, int64_t k) { return (size_t)(m * k / 32) * 6u; }

/* One block: 32 floats -> the 32-bit code word and the fp16 scale bits. */
int oracle_q1_0_quantize_block(const float *w, uint32_t *bits, uint16_t *d_bits)
{
    double sum = 0.0;
    for (int i = 0; i < 32; i++) {
        if (!isfinite(w[i])) return ORACLE_ENONFINITE;
        sum += fabs((double)w[i]);
    }
    uint16_t dh = oracle_f64_to_fp16(sum / 32.0);
    if ((dh & 0x7C00) == 0x7C00) return ORACLE_ERANGE; /* scale not finite in fp16 */
    uint32_t word = 0;
    for (int i = 0; i < 32; i++)
        if (w[i] >= 0.0f) word |= (uint32_t)1 << i;
    *bits = word;
    *d_bits = dh;
    return ORACLE_OK;
}

int oracle_q1_0_quantize(const float *w, int64_t m, int64_t k, uint8_t *out)
{
    if (m < 0 || k <= 0 || k % 32 != 0) return ORACLE_EINVAL;
    int64_t nb = k / 32;
    uint8_t *scales = out + (size_t)(m * k / 8);
    for (int64_t r = 0; r < m; r++) {
        for (int64_t b = 0; b < nb; b++) {
            uint32_t word;
            uint16_t dh;
            int st = oracle_q1_0_quantize_block(w + r * k + b * 32, &word, &dh);
            if (st != ORACLE_OK) return st;
            uint8_t *o = out + (r * nb + b) * 4;
            for (int j = 0; j < 4; j++) o[j] = (uint8_t)(word >> (8 * j));
            scales[(r * nb + b) * 2] = (uint8_t)(dh & 0xFF);
            scales[(r * nb + b) * 2 + 1] = (uint8_t)(dh >> 8);
        }
    }
    return ORACLE_OK;
}

/* Dequantized weight (r, c): +d or -d, exact in binary32. */
float oracle_q1_0_weight(const uint8_t *buf, int64_t m, int64_t k, int64_t r, int64_t c)
{
    int64_t nb = k / 32;
    int64_t b = c / 32;
    int e = (int)(c % 32);
    int bit = (buf[(r * nb + b) * 4 + e / 8] >> (e % 8)) & 1;
    const uint8_t *s = buf + (size_t)(m * k / 8) + (r * nb + b) * 2;
    float d = oracle_fp16_to_fp32((uint16_t)(s[0] | (s[1] << 8)));
    return bit ? d : -d;
}

void oracle_q1_0_dequantize(const uint8_t *buf, int64_t m, int64_t k, float *w_hat)
{
    for (int64_t r = 0; r < m; r++)
        for (int64_t c = 0; c < k; c++)
            w_hat[r * k + c] = oracle_q1_0_weight(buf, m, k, r, c);
}

/* ------------------------------------------------------------------------
 * Q2_K (llama.cpp's 2-bit K-quant, the q2_k of the technical summary's
 * results): 256-weight super-blocks of sixteen 16-weight sub-blocks; per
 * sub-block a 4-bit scale sc and a 4-bit min m (one byte: sc low nibble,
 * m high nibble); per super-block fp16 d and dmin; 2-bit codes q; value
 * d*sc*q - dmin*m. The same fields as llama.cpp's 84-byte block, stored in
 * three planes so that every field is naturally aligned:
 *   bytes [0, m*k/4)                code plane: super-block (r, s) at
 *       (r*ns + s)*64; the code of its element e is bits 2j, 2j+1 of byte
 *       32*(e/128) + e%32, j = (e%128)/32 (llama.cpp's order);
 *   bytes [m*k/4, m*k*5/16)         scale plane: byte e/16 of super-block
 *       (r, s) at m*k/4 + (r*ns + s)*16;
 *   bytes [m*k*5/16, m*k*21/64)     fp16 d then fp16 dmin of super-block
 *       (r, s) at m*k*5/16 + (r*ns + s)*4, little-endian.
 * ------------------------------------------------------------------------ */

size_t oracle_q2_k_bytes(int64_t m, int64_t k) { return (size_t)(m * (k / 256)) * 84u; }

/* Min/max quantizer for one super-block, in float64 (the Q4_K reading with
 * 2-bit codes and 4-bit scales):
 *   per 16-weight sub-block: lo = min(0, min w), hi = max w, s = (hi - lo)/3, mu = -lo
 *   d = fp16(max s / 15), dmin = fp16(max mu / 15)
 *   sc = clamp(round(s/d), 0, 15), m = clamp(round(mu/dmin), 0, 15)
 *   q = clamp(round((w + dmin*m) / (d*sc)), 0, 3)   (0 where a divisor is 0)
 * Writes the 64 code bytes, 16 scale bytes and 4 bytes of d, dmin. */
int oracle_q2_k_quantize_superblock(const float *w, uint8_t *codes, uint8_t *scales, uint8_t *dd)
{
    double s[16], mu[16];
    double smax = 0.0, mumax = 0.0;
    for (int i = 0; i < 256; i++)
        if (!isfinite(w[i])) return ORACLE_ENONFINITE;
    for (int j = 0; j < 16; j++) {
        double lo = 0.0, hi = (double)w[16 * j];
        for (int i = 0; i < 16; i++) {
            double v = (double)w[16 * j + i];
            if (v < lo) lo = v;
            if (v > hi) hi = v;
        }
        s[j] = (hi - lo) / 3.0;
        mu[j] = -lo;
        if (s[j] > smax) smax = s[j];
        if (mu[j] > mumax) mumax = mu[j];
    }
    uint16_t dh = oracle_f64_to_fp16(smax / 15.0);
    uint16_t mh = oracle_f64_to_fp16(mumax / 15.0);
    if ((dh & 0x7C00) == 0x7C00 || (mh & 0x7C00) == 0x7C00) return ORACLE_ERANGE;
    double d = (double)oracle_fp16_to_fp32(dh);
    double dmin = (double)oracle_fp16_to_fp32(mh);
    int sc[16], mn[16];
    for (int j = 0; j < 16; j++) {
        sc[j] = d == 0.0 ? 0 : clampi((int)round_half_away(s[j] / d), 0, 15);
        mn[j] = dmin == 0.0 ? 0 : clampi((int)round_half_away(mu[j] / dmin), 0, 15);
        scales[j] = (uint8_t)(sc[j] | (mn[j] << 4));
    }
    for (int b = 0; b < 64; b++) codes[b] = 0;
    for (int e = 0; e < 256; e++) {
        int j = e / 16;
        double step = d * (double)sc[j];
        double off = dmin * (double)mn[j];
        int q = step == 0.0 ? 0 : clampi((int)round_half_away(((double)w[e] + off) / step), 0, 3);
        codes[32 * (e / 128) + e % 32] |= (uint8_t)(q << (2 * ((e % 128) / 32)));
    }
    dd[0] = (uint8_t)(dh & 0xFF);
    dd[1] = (uint8_t)(dh >> 8);
    dd[2] = (uint8_t)(mh & 0xFF);
    dd[3] = (uint8_t)(mh >> 8);
    return ORACLE_OK;
}

int oracle_q2_k_quantize(const float *w, int64_t m, int64_t k, uint8_t *out)
{
    if (m < 0 || k <= 0 || k % 256 != 0) return ORACLE_EINVAL;
    int64_t ns = k / 256;
    uint8_t *scales = out + (size_t)(m * k / 4);
    uint8_t *dd = out + (size_t)(m * k / 4 + m * k / 16);
    for (int64_t r = 0; r < m; r++)
        for (int64_t sb = 0; sb < ns; sb++) {
            int64_t i = r * ns + sb;
            int st = oracle_q2_k_quantize_superblock(w + r * k + sb * 256, out + i * 64, scales + i * 16, dd + i * 4);
            if (st != ORACLE_OK) return st;
        }
    return ORACLE_OK;
}

/* Dequantized weight (r, c): (d*sc)*q - dmin*m in binary32; both products are
 * exact (at most 17 and 15 significant bits), the subtraction rounds once. */
float oracle_q2_k_weight(const uint8_t *buf, int64_t m, int64_t k, int64_t r, int64_t c)
{
    int64_t ns = k / 256;
    int64_t i = r * ns + c / 256;
    int e = (int)(c % 256);
    uint8_t byte = buf[i * 64 + 32 * (e / 128) + e % 32];
    int q = (byte >> (2 * ((e % 128) / 32))) & 3;
    uint8_t scm = buf[(size_t)(m * k / 4) + i * 16 + e / 16];
    const uint8_t *dd = buf + (size_t)(m * k / 4 + m * k / 16) + i * 4;
    float d = oracle_fp16_to_fp32((uint16_t)(dd[0] | (dd[1] << 8)));
    float dmin = oracle_fp16_to_fp32((uint16_t)(dd[2] | (dd[3] << 8)));
    float a = (d * (float)(scm & 15)) * (float)q;
    float b = dmin * (float)(scm >> 4);
    return a - b;
}

void oracle_q2_k_dequantize(const uint8_t *buf, int64_t m, int64_t k, float *w_hat)
{
    for (int64_t r = 0; r < m; r++)
        for (int64_t c = 0; c < k; c++)
            w_hat[r * k + c] = oracle_q2_k_weight(buf, m, k, r, c);
}

/* ------------------------------------------------------------------------
 * Q4_K.  Buffer: m * (k/256) super-blocks of 144 bytes, row-major:
 *   [0,2) fp16 d   [2,4) fp16 dmin   [4,16) twelve bytes S holding eight
 *   6-bit scales and eight 6-bit mins   [16,144) 128 nibble bytes.
 * 6-bit packing (llama.cpp's K-quant packing as publicly described):
 *   sub-block j < 4 : scale = S[j] & 63,   min = S[j+4] & 63
 *   sub-block j >= 4: scale = (S[j+4] & 15) | ((S[j-4] >> 6) << 4)
 *                     min   = (S[j+4] >> 4) | ((S[j]   >> 6) << 4)
 * Nibbles: 4 chunks of 32 bytes; in chunk c, byte i holds weight 64c+i in its
 * low nibble (sub-block 2c) and weight 64c+32+i in its high nibble (2c+1).
 * ------------------------------------------------------------------------ */

size_t oracle_q4_k_bytes(int64_t m, int64_t k) { return (size_t)(m * (k / 256)) * 144u; }

void oracle_q4_k_unpack_scales(const uint8_t *S, uint8_t *sc, uint8_t *mn)
{
    for (int j = 0; j < 8; j++) {
        if (j < 4) {
            sc[j] = S[j] & 63;
            mn[j] = S[j + 4] & 63;
        } else {
            sc[j] = (uint8_t)((S[j + 4] & 15) | ((S[j - 4] >> 6) << 4));
            mn[j] = (uint8_t)((S[j + 4] >> 4) | ((S[j] >> 6) << 4));
        }
    }
}

void oracle_q4_k_pack_scales(const uint8_t *sc, const uint8_t *mn, uint8_t *S)
{
    for (int j = 0; j < 12; j++) S[j] = 0;
    for (int j = 0; j < 8; j++) {
        if (j < 4) {
            S[j] |= (uint8_t)(sc[j] & 63);
            S[j + 4] |= (uint8_t)(mn[j] & 63);
        } else {
            S[j + 4] |= (uint8_t)((sc[j] & 15) | ((mn[j] & 15) << 4));
            S[j - 4] |= (uint8_t)((sc[j] >> 4) << 6);
            S[j] |= (uint8_t)((mn[j] >> 4) << 6);
        }
    }
}

/* Min/max quantizer for one super-block (256 floats -> 144 bytes), in float64:
 *   per sub-block: lo = min(0, min w), hi = max w, s = (hi - lo)/15, mu = -lo
 *   d = fp16(max s / 63), dmin = fp16(max mu / 63)
 *   sc = clamp(round(s/d), 0, 63), m = clamp(round(mu/dmin), 0, 63)
 *   q = clamp(round((w + dmin*m) / (d*sc)), 0, 15)   (0 where a divisor is 0) */
int oracle_q4_k_quantize_superblock(const float *w, uint8_t *out)
{
    double s[8], mu[8];
    double smax = 0.0, mumax = 0.0;
    for (int i = 0; i < 256; i++)
        if (!isfinite(w[i])) return ORACLE_ENONFINITE;
    for (int j = 0; j < 8; j++) {
        double lo = 0.0, hi = (double)w[32 * j];
        for (int i = 0; i < 32; i++) {
            double v = (double)w[32 * j + i];
            if (v < lo) lo = v;
            if (v > hi) hi = v;
        }
        s[j] = (hi - lo) / 15.0;
        mu[j] = -lo;
        if (s[j] > smax) smax = s[j];
        if (mu[j] > mumax) mumax = mu[j];
    }
    uint16_t dh = oracle_f64_to_fp16(smax / 63.0);
    uint16_t mh = oracle_f64_to_fp16(mumax / 63.0);
    if ((dh & 0x7C00) == 0x7C00 || (mh & 0x7C00) == 0x7C00) return ORACLE_ERANGE;
    double d = (double)oracle_fp16_to_fp32(dh);
    double dmin = (double)oracle_fp16_to_fp32(mh);
    uint8_t sc[8], mn[8];
    for (int j = 0; j < 8; j++) {
        sc[j] = (uint8_t)(d == 0.0 ? 0 : clampi((int)round_half_away(s[j] / d), 0, 63));
        mn[j] = (uint8_t)(dmin == 0.0 ? 0 : clampi((int)round_half_away(mu[j] / dmin), 0, 63));
    }
    uint8_t q[256];
    for (int j = 0; j < 8; j++) {
        double step = d * (double)sc[j];
        double off = dmin * (double)mn[j];
        for (int i = 0; i < 32; i++) {
            double v = (double)w[32 * j + i];
            q[32 * j + i] = (uint8_t)(step == 0.0 ? 0 : clampi((int)round_half_away((v + off) / step), 0, 15));
        }
    }
    out[0] = (uint8_t)(dh & 0xFF);
    out[1] = (uint8_t)(dh >> 8);
    out[2] = (uint8_t)(mh & 0xFF);
    out[3] = (uint8_t)(mh >> 8);
    oracle_q4_k_pack_scales(sc, mn, out + 4);
    for (int c = 0; c < 4; c++)
        for (int i = 0; i < 32; i++)
            out[16 + 32 * c + i] = (uint8_t)(q[64 * c + i] | (q[64 * c + 32 + i] << 4));
    return ORACLE_OK;
}

int oracle_q4_k_quantize(const float *w, int64_t m, int64_t k, uint8_t *out)
{
    if (m < 0 || k <= 0 || k % 256 != 0) return ORACLE_EINVAL;
    int64_t ns = k / 256;
    for (int64_t r = 0; r < m; r++)
        for (int64_t sb = 0; sb < ns; sb++) {
            int st = oracle_q4_k_quantize_superblock(w + r * k + sb * 256, out + (r * ns + sb) * 144);
            if (st != ORACLE_OK) return st;
        }
    return ORACLE_OK;
}

/* Dequantized weight (r, c): (d*sc)*q - dmin*m in binary32.  Both products are
 * exact (at most 21 significant bits), so the subtraction is the one rounding. */
float oracle_q4_k_weight(const uint8_t *buf, int64_t m, int64_t k, int64_t r, int64_t c)
{
    (void)m;
    int64_t ns = k / 256;
    const uint8_t *sbp = buf + (r * ns + c / 256) * 144;
    int e = (int)(c % 256);
    int j = e / 32;                  /* sub-block */
    int chunk = e / 64;
    int i = e % 32;
    int hi = (e % 64) >= 32;
    uint8_t byte = sbp[16 + 32 * chunk + i];
    int q = hi ? (byte >> 4) : (byte & 15);
    uint8_t sc[8], mn[8];
    oracle_q4_k_unpack_scales(sbp + 4, sc, mn);
    float d = oracle_fp16_to_fp32((uint16_t)(sbp[0] | (sbp[1] << 8)));
    float dmin = oracle_fp16_to_fp32((uint16_t)(sbp[2] | (sbp[3] << 8)));
    float a = (d * (float)sc[j]) * (float)q;
    float b = dmin * (float)mn[j];
    return a - b;
}

void oracle_q4_k_dequantize(const uint8_t *buf, int64_t m, int64_t k, float *w_hat)
{
    for (int64_t r = 0; r < m; r++)
        for (int64_t c = 0; c < k; c++)
            w_hat[r * k + c] = oracle_q4_k_weight(buf, m, k, r, c);
}

/* ------------------------------------------------------------------------
 * Products.  fmt 0 = Q4_0, 1 = Q4_K.  Rows [row0, row1) only, so a caller
 * may split the rows across threads; the arithmetic does not change.
 *
 * matvec: y[t][i] = fp32( sum_k w_hat[i][k] * x[t][k] ), the sum taken in
 *         float64 over ascending k (every product is exact in float64).
 * matmul: Y[t][i] = fp32( sum_k w_eff[i][k] * X[t][k] ) with X in bf16 and
 *         w_eff = w_hat, or bf16_RNE(w_hat) when round_w_bf16 is set.
 * ------------------------------------------------------------------------ */

static float weight_at(int fmt, const uint8_t *w, int64_t m, int64_t k, int64_t r, int64_t c)
{
    if (fmt == 0) return oracle_q4_0_weight(w, m, k, r, c);
    if (fmt == 2) return oracle_q8_0_weight(w, m, k, r, c);
    if (fmt == 3) return oracle_q2_k_weight(w, m, k, r, c);
    if (fmt == 4) return oracle_q1_0_weight(w, m, k, r, c);
    return oracle_q4_k_weight(w, m, k, r, c);
}

void oracle_matvec(int fmt, const uint8_t *w, int64_t m, int64_t k,
                   const float *x, int64_t n, float *y, int64_t row0, int64_t row1)
{
    for (int64_t i = row0; i < row1; i++) {
        for (int64_t t = 0; t < n; t++) {
            double acc = 0.0;
            for (int64_t c = 0; c < k; c++)
                acc += (double)weight_at(fmt, w, m, k, i, c) * (double)x[t * k + c];
            y[t * m + i] = (float)acc;
        }
    }
}

/* Same as oracle_matvec but also returns sum_k |w_hat * x| per output, the
 * scale against which an elementwise forward error is measured. */
void oracle_matvec_absdot(int fmt, const uint8_t *w, int64_t m, int64_t k,
                          const float *x, int64_t n, float *y, double *absdot,
                          int64_t row0, int64_t row1)
{
    for (int64_t i = row0; i < row1; i++) {
        for (int64_t t = 0; t < n; t++) {
            double acc = 0.0, aacc = 0.0;
            for (int64_t c = 0; c < k; c++) {
                double p = (double)weight_at(fmt, w, m, k, i, c) * (double)x[t * k + c];
                acc += p;
                aacc += fabs(p);
            }
            y[t * m + i] = (float)acc;
            absdot[t * m + i] = aacc;
        }
    }
}

void oracle_matmul(int fmt, const uint8_t *w, int64_t m, int64_t k,
                   const uint16_t *x_bf16, int64_t n, float *y, int round_w_bf16,
                   double *absdot, int64_t row0, int64_t row1)
{
    for (int64_t i = row0; i < row1; i++) {
        for (int64_t t = 0; t < n; t++) {
            double acc = 0.0, aacc = 0.0;
            for (int64_t c = 0; c < k; c++) {
                float wv = weight_at(fmt, w, m, k, i, c);
                if (round_w_bf16) wv = oracle_bf16_to_fp32(oracle_fp32_to_bf16(wv));
                double p = (double)wv * (double)oracle_bf16_to_fp32(x_bf16[t * k + c]);
                acc += p;
                aacc += fabs(p);
            }
            y[t * m + i] = (float)acc;
            if (absdot) absdot[t * m + i] = aacc;
        }
    }
}

/* Magnitude scale of the terms a format's value is built from, summed with
 * |x|: Q4_0's value is the single term (q - 8)*d, so the scale is
 * sum_k |w_hat * x|; Q4_K's value is the difference d*sc*q - dmin*m of two
 * terms, so the scale is sum_k (|d*sc*q| + |dmin*m|) * |x|. An elementwise
 * forward-error bound for an evaluation that keeps the two Q4_K terms apart
 * (as the format's structure invites) is stated against this scale. */
static double term_magnitude(int fmt, const uint8_t *w, int64_t m, int64_t k, int64_t r, int64_t c)
{
    if (fmt == 0) return fabs((double)oracle_q4_0_weight(w, m, k, r, c));
    if (fmt == 2) return fabs((double)oracle_q8_0_weight(w, m, k, r, c));
    if (fmt == 4) return fabs((double)oracle_q1_0_weight(w, m, k, r, c));
    if (fmt == 3) {
        int64_t i = r * (k / 256) + c / 256;
        int e = (int)(c % 256);
        int q = (w[i * 64 + 32 * (e / 128) + e % 32] >> (2 * ((e % 128) / 32))) & 3;
        uint8_t scm = w[(size_t)(m * k / 4) + i * 16 + e / 16];
        const uint8_t *dd = w + (size_t)(m * k / 4 + m * k / 16) + i * 4;
        double d = oracle_fp16_to_fp32((uint16_t)(dd[0] | (dd[1] << 8)));
        double dmin = oracle_fp16_to_fp32((uint16_t)(dd[2] | (dd[3] << 8)));
        return fabs(d * (scm & 15) * q) + fabs(dmin * (scm >> 4));
    }
    int64_t ns = k / 256;
    const uint8_t *sbp = w + (r * ns + c / 256) * 144;
    int e = (int)(c % 256);
    int j = e / 32;
    uint8_t byte = sbp[16 + 32 * (e / 64) + e % 32];
    int q = ((e % 64) >= 32) ? (byte >> 4) : (byte & 15);
    uint8_t sc[8], mn[8];
    oracle_q4_k_unpack_scales(sbp + 4, sc, mn);
    double d = oracle_fp16_to_fp32((uint16_t)(sbp[0] | (sbp[1] << 8)));
    double dmin = oracle_fp16_to_fp32((uint16_t)(sbp[2] | (sbp[3] << 8)));
    return fabs(d * sc[j] * q) + fabs(dmin * mn[j]);
}

void oracle_matvec_termscale(int fmt, const uint8_t *w, int64_t m, int64_t k, const float *x, int64_t n,
                             double *scale, int64_t row0, int64_t row1)
{
    for (int64_t i = row0; i < row1; i++)
        for (int64_t t = 0; t < n; t++) {
            double acc = 0.0;
            for (int64_t c = 0; c < k; c++) acc += term_magnitude(fmt, w, m, k, i, c) * fabs((double)x[t * k + c]);
            scale[t * m + i] = acc;
        }
}

/* Gated decode product (the gate and up projections of a gated MLP fused into
 * one launch, the activation applied to the gate; kernel fusion: WebGPT
 * README, "Roadmap"; Llamas on the Web technical summary, "Experimental
 * results"). The matrix has 2m rows: gate rows 0..m-1, then up rows
 * m..2m-1. With g and u the fp64 row products (as in oracle_matvec, before
 * any rounding), y[t][i] = fp32( silu(g) * u ), silu(g) = g / (1 + exp(-g)),
 * evaluated in fp64. g and u are also returned (fp64) when the pointers are
 * not null. Rows [row0, row1) of the output. */
void oracle_matvec_silu_mul(int fmt, const uint8_t *w, int64_t m, int64_t k, const float *x, int64_t n,
                            float *y, double *g_out, double *u_out, int64_t row0, int64_t row1)
{
    for (int64_t i = row0; i < row1; i++) {
        for (int64_t t = 0; t < n; t++) {
            double g = 0.0, u = 0.0;
            for (int64_t c = 0; c < k; c++) {
                g += (double)weight_at(fmt, w, 2 * m, k, i, c) * (double)x[t * k + c];
                u += (double)weight_at(fmt, w, 2 * m, k, m + i, c) * (double)x[t * k + c];
            }
            double silu = g / (1.0 + exp(-g));
            y[t * m + i] = (float)(silu * u);
            if (g_out) g_out[t * m + i] = g;
            if (u_out) u_out[t * m + i] = u;
        }
    }
}

/* One output of the products, for sampled checks at full size. */
double oracle_matvec_one(int fmt, const uint8_t *w, int64_t m, int64_t k,
                         const float *x, int64_t t, int64_t i, double *absdot)
{
    double acc = 0.0, aacc = 0.0;
    for (int64_t c = 0; c < k; c++) {
        double p = (double)weight_at(fmt, w, m, k, i, c) * (double)x[t * k + c];
        acc += p;
        aacc += fabs(p);
    }
    if (absdot) *absdot = aacc;
    return acc;
}
