/*
 * q4.h -- C ABI of the Q4 weight-matrix product library for AMD Instinct
 * MI355X (gfx950).
 *
 * What the library computes: the matrix products of LLM decode and prefill
 * with weights block-quantized to 4 bits, dequantized inside the product --
 * in registers for the decode matrix-vector product, through shared memory
 * (LDS) for the prefill matrix-matrix product (Llamas on the Web, technical
 * summary, Methodology section 3, "integrated dequantization"). Weight
 * formats are flat byte buffers decoded by a per-format routine chosen at
 * compile time (same section, "extensibility"); all memory is allocated by
 * the caller ahead of time (Methodology section 1, "static allocation").
 *
 * Conventions for every entry point:
 *   - The caller owns every buffer. The library allocates no memory. What it
 *     keeps between calls per device: cached device attributes (compute
 *     units, the workgroup LDS limit), once per device and kernel the opt-in
 *     of kernels that use more than 64 KiB of LDS, and the device address of
 *     the static 256 KiB array that q4_llama_step_noalloc works in (loaded
 *     with the library's code, written only by that call); the graph handles
 *     below are caller-owned state. Calls are reentrant, except that calls of
 *     q4_llama_step_noalloc that overlap on one GPU share its array.
 *   - Matrices are row-major. W is logically [m][k] (k = input dimension,
 *     m = output dimension), quantized along k. Activations are token-major:
 *     x[n][k], y[n][m].
 *   - Device entry points validate every argument first. On any error they
 *     return a negative status, enqueue nothing and leave y untouched; only
 *     then do they make a HIP call. Faults during execution surface at the
 *     caller's next synchronization.
 *   - Device work is enqueued on the given HIP stream (NULL = null stream);
 *     the call returns without synchronizing.
 *   - No exception or abort crosses the ABI.
 *
 * Weight buffer layouts (produced by q4_quantize_ref):
 *   Q4_0, m x k, k % 32 == 0, m*k*9/16 bytes, "plane-split":
 *     bytes [0, m*k/2): nibble plane. Block (r, b) (row r, weights
 *       32b..32b+31) occupies 16 bytes at (r*k/32 + b)*16; byte j holds the
 *       code of weight j in its low nibble and of weight j+16 in its high
 *       nibble (llama.cpp's order inside a block).
 *     bytes [m*k/2, m*k*9/16): scale plane. The fp16 scale d of block (r, b)
 *       is at m*k/2 + (r*k/32 + b)*2, little-endian.
 *     Weight value: (q - 8) * d. This moves the same bytes as llama.cpp's
 *     18-byte array-of-blocks layout, but every 16-byte group is 16-byte
 *     aligned for 128-bit loads.
 *   Q4_K, m x k, k % 256 == 0, m*(k/256)*144 bytes: row-major 144-byte
 *     super-blocks of 256 weights: [0,2) fp16 d, [2,4) fp16 dmin, [4,16)
 *     twelve bytes S packing eight 6-bit scales sc and eight 6-bit mins mn
 *     (sub-block j < 4: sc = S[j] & 63, mn = S[j+4] & 63; j >= 4:
 *     sc = (S[j+4] & 15) | (S[j-4] >> 6) << 4, mn = (S[j+4] >> 4) |
 *     (S[j] >> 6) << 4), [16,144) nibbles: four 32-byte chunks; byte i of
 *     chunk c holds weight 64c+i (low nibble) and 64c+32+i (high nibble).
 *     Weight value of sub-block j: d*sc_j*q - dmin*mn_j.
 *   Q8_0, m x k, k % 32 == 0, m*k*17/16 bytes, plane-split like Q4_0:
 *     bytes [0, m*k): code plane. Block (r, b) occupies 32 bytes at
 *       (r*k/32 + b)*32; byte j is the code of weight j, two's complement.
 *     bytes [m*k, m*k*17/16): scale plane, fp16 d of block (r, b) at
 *       m*k + (r*k/32 + b)*2, little-endian.
 *     Weight value: q * d. (The 8-bit format the technical summary's results
 *     compare with q4_k_m and q2_k: "Experimental results", quantization
 *     impact.)
 *   Q2_K, m x k, k % 256 == 0, m*(k/256)*84 bytes: the fields of llama.cpp's
 *     84-byte 2-bit K-quant block in three planes (ns = k/256 super-blocks
 *     per row, super-block (r, s) has index i = r*ns + s):
 *     bytes [0, m*k/4): code plane, 64 bytes per super-block at i*64; the
 *       2-bit code of its element e is bits 2j, 2j+1 of byte
 *       32*(e/128) + e%32, j = (e%128)/32.
 *     bytes [m*k/4, m*k*5/16): scale plane, 16 bytes per super-block at
 *       m*k/4 + i*16; byte e/16 holds the 4-bit scale sc (low nibble) and
 *       4-bit min mn (high nibble) of element e's 16-weight sub-block.
 *     bytes [m*k*5/16, m*k*21/64): fp16 d then fp16 dmin at m*k*5/16 + i*4.
 *     Weight value: d*sc*q - dmin*mn.
 *   Q1_0, m x k, k % 32 == 0, m*k*3/16 bytes, plane-split like Q4_0:
 *     bytes [0, m*k/8): bit plane. Block (r, b) occupies a 32-bit
 *       little-endian word at (r*k/32 + b)*4; bit e is the code b_e of
 *       weight e of the block.
 *     bytes [m*k/8, m*k*3/16): scale plane, fp16 d of block (r, b) at
 *       m*k/8 + (r*k/32 + b)*2, little-endian.
 *     Weight value: (2 b_e - 1) * d, i.e. +d or -d. (The technical summary
 *     names q1_0 only as a 1-bit format that is added by writing one
 *     dequantization routine: Methodology section 3, extensibility. This is
 *     the Q4_0 block with a one-bit code.)
 */
#ifndef Q4_H
#define Q4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Weight formats: legacy Q4_0 and Q8_0 and the K-quants Q4_K and Q2_K
 * (llama.cpp families the technical summary names: problem statement item 3;
 * q8_0, q4_k_m and q2_k in its results), and the 1-bit Q1_0 (its
 * extensibility example). */
typedef enum { Q4_FMT_Q4_0 = 0, Q4_FMT_Q4_K = 1, Q4_FMT_Q8_0 = 2, Q4_FMT_Q2_K = 3, Q4_FMT_Q1_0 = 4 } q4_format;

/* Status codes. */
enum {
    Q4_OK = 0,
    Q4_EINVAL = -1,       /* bad size, null pointer, k not a whole number of blocks, short buffer */
    Q4_EUNSUPPORTED = -2, /* n outside 1..8 for gemv; unknown format; w, x or y of 2 GiB or more */
    Q4_EALIGN = -3,       /* w not 16-byte aligned; x or y not 4-byte aligned */
    Q4_ENONFINITE = -4,   /* NaN or Inf among the weights given to the quantizer */
    Q4_ERANGE = -5,       /* a block scale that rounds to a non-finite fp16 */
    Q4_EHIP = -6          /* the HIP runtime reported a launch or capture error */
};

/* Bytes of the quantized buffer for an m x k matrix; 0 if k is not a
 * positive multiple of the block (32 for Q4_0, Q8_0 and Q1_0, 256 for the K-quants),
 * m < 0, or the format is unknown. Host only; no device work. (Q4_0 stores
 * 16-bit weights in 4 bits per parameter plus a shared fp16 scale per 32:
 * MicroLLM Lab post, "Seven models, all in Q4", and the block sizes of the
 * llama.cpp formats the technical summary of Llamas on the Web serves,
 * problem statement.) */
size_t q4_weight_bytes(int fmt, int64_t m, int64_t k);

/* Host quantizer: float32 W[m][k] (host memory) -> packed buffer `out`
 * (host memory, at least q4_weight_bytes(fmt, m, k) bytes).
 * Q4_0 block: d = fp16_rne(max|w| / 7) (binary32 division); codes
 *   q = clamp(round_half_away(w / d) + 8, 0, 15), all 8 when d == 0.
 * Q4_K super-block (min/max reading, evaluated in float64): per sub-block
 *   lo = min(0, min w), hi = max w, s = (hi - lo)/15, mu = -lo;
 *   d = fp16_rne(max s / 63), dmin = fp16_rne(max mu / 63);
 *   sc = clamp(round_half_away(s/d), 0, 63), mn = clamp(round_half_away(mu/dmin), 0, 63);
 *   q = clamp(round_half_away((w + dmin*mn)/(d*sc)), 0, 15) (0 where a divisor is 0).
 * Q8_0 block: d = fp16_rne(max|w| / 127) (binary32 division); codes
 *   q = clamp(round_half_away(w / d), -127, 127), all 0 when d == 0.
 * Q2_K super-block: the Q4_K reading with 16-weight sub-blocks, s = (hi - lo)/3,
 *   d = fp16_rne(max s / 15), dmin = fp16_rne(max mu / 15), 4-bit sc and mn
 *   (clamp 0..15) and 2-bit codes (clamp 0..3).
 * Q1_0 block: d = fp16_rne(sum|w| / 32) (float64 sum and quotient, one
 *   rounding: the least-squares scale for codes of fixed sign); codes
 *   b = 1 for w >= 0 (either zero included), 0 for w < 0.
 * Blocks are quantized row by row; the status is that of the first failing
 * block in row-major order (Q4_ENONFINITE for NaN/Inf, Q4_ERANGE for a scale
 * that overflows fp16), and `out` is then unspecified.
 * (16-bit weights to 4 bits per parameter: MicroLLM Lab post, "Seven models,
 * all in Q4".) */
int q4_quantize_ref(int fmt, const float *w, int64_t m, int64_t k, void *out, size_t out_bytes);

/* Decode product y[t][i] = sum_k w_hat[i][k] * x[t][k] for t < n, fp32 out
 * (Llamas on the Web, technical summary, problem statement: the product of a
 * matrix in a llama.cpp quantization format with an activation vector).
 * w: device, quantized as above, 16-byte aligned; x: device float32 [n][k],
 * 4-byte aligned; y: device float32 [n][m], 4-byte aligned, fully written.
 * n must be 1..8 (decode batch); m == 0 is a successful no-op.
 * Weights are dequantized in registers and never written back (Llamas on the
 * Web, technical summary, Methodology section 3). Each 32-element piece of x
 * is scaled exactly by a power of two (its largest magnitude into
 * [2^14, 2^15)), then held as a pair of fp16 values hi + lo (about 2^-23
 * relative) when m < 256, or as one fp16 value when m >= 256 (round to
 * nearest: at most 2^-11 relative, so every output is within
 * 2^-11 * sum_k |w_hat[i][k] x[t][k]| plus the fp32 sums' rounding); the
 * weight codes are exact fp16 values, products and sums are fp32. A NaN among
 * token t's activations makes every y[t][i] NaN, as exact IEEE evaluation
 * does (0 * NaN included); the other tokens are unaffected. x is otherwise
 * expected finite. One token on a matrix of rows of up to 14560 weights
 * runs the streaming kernel, Q4_K at several tokens on 256 rows or more the
 * matrix-core kernel (from 3 tokens on, and at 2 tokens on rows of up to
 * 2048 weights), everything else the tiled
 * kernel (see q4_gemv_tuning); all
 * are deterministic. The matrix-core kernel scales each 256-element piece of
 * a token's x (one Q4_K super-block) by a power of two into [2^14, 2^15) and
 * rounds it to one fp16 value (the same 2^-11 bound); its codes sc*q and
 * mins are exact fp16 values and its products and sums fp32. */
int q4_gemv(int fmt, const void *w, const float *x, float *y,
            int64_t m, int64_t k, int64_t n, void *hip_stream);

/* Gated decode product: the gate and up projections of a gated MLP in one
 * launch, with the activation applied to the gate (kernels fused: WebGPT
 * README, "Roadmap"; the technical summary of Llamas on the Web credits fused
 * kernels for prefill throughput, "Experimental results"). w is one quantized
 * (2m) x k matrix, gate rows 0..m-1 then up rows m..2m-1, in the layout of
 * q4_quantize_ref for 2m rows (quantize the stacked matrix). For t < n and
 * i < m:
 *   y[t][i] = silu(g) * u,  g = sum_k w_hat[i][k] x[t][k],
 *   u = sum_k w_hat[m+i][k] x[t][k],  silu(g) = g / (1 + exp(-g)).
 * g and u are summed exactly as q4_gemv_tuned sums the rows of the stacked
 * matrix with the kernel the gated product shares (same arithmetic, same
 * tolerance): the matrix-core kernel for Q4_K where q4_gemv would pick it for
 * the stacked matrix and the row has at most 4096 weights, else the tiled
 * kernel (Q4_GEMV_KERNEL_TILED); the epilogue is fp32. x [n][k] and y [n][m]
 * are device arrays, n is 1..8. Errors as q4_gemv, with the size limits
 * applying to the 2m-row matrix (m below 2^29). */
int q4_gemv_glu(int fmt, const void *w, const float *x, float *y,
                int64_t m, int64_t k, int64_t n, void *hip_stream);

/* One-token decode product with the residual add and RMSNorm of its input
 * fused into the launch (the normalisation ahead of each projection block of
 * a Llama-family model, the family of the SmolLM2 models the MicroLLM Lab post
 * runs; fused kernels: WebGPT README, "Roadmap"). With v = x + delta (v = x if
 * delta is NULL) and h = v / sqrt(mean(v^2) + eps) * gain:
 *   epilogue Q4_EPILOGUE_NONE:     y = W h, W of m rows (as q4_gemv, n = 1);
 *   epilogue Q4_EPILOGUE_SILU_MUL: y = silu(W_gate h) * (W_up h), W of 2m
 *     rows (as q4_gemv_glu, n = 1);
 * and, if x_out is not NULL, x_out = v (the updated residual stream).
 * The kernel stages v * gain and scales each reduced row sum by the fp32
 * factor 1/sqrt(mean(v^2) + eps) (the same value for every row), so the
 * product's tolerance is q4_gemv's, relative to the normalised input.
 * x: device float32 [k], 4-byte aligned; delta, gain, x_out: device float32
 * [k], 16-byte aligned; x_out must not
 * overlap x, delta or y (it is written while they are read). y: device
 * float32 [m]. k at most 14560 (the whole row is staged in one workgroup's
 * LDS). m == 0 is a successful no-op that writes nothing (x_out included).
 * Errors as q4_gemv / q4_gemv_glu, plus Q4_EINVAL for a NULL gain, an
 * eps that is negative, infinite or NaN, an overlapping x_out or an unknown
 * epilogue, Q4_EALIGN for a misaligned delta, gain or x_out and
 * Q4_EUNSUPPORTED for a longer row. */
int q4_gemv_addnorm(int fmt, const void *w, const float *x, const float *delta, const float *gain, float eps,
                    float *x_out, float *y, int64_t m, int64_t k, int epilogue, void *hip_stream);

/* Kernel and geometry of the decode product. The library picks them per
 * shape; the tuned entry point lets a sweep override them (tile and
 * workgroup sizes are tunable parameters whose defaults come from an
 * empirical sweep: Llamas on the Web, technical summary, Methodology
 * section 2, "tunable parameters"). A zero field keeps the library's choice.
 * Two kernels:
 *   Q4_GEMV_KERNEL_TILED: workgroups stride over tiles of rows, staging the
 *     activations per workgroup; any n. Instantiated geometries
 *     (lanes_per_row, rows_per_lane, waves_per_group): (8,1,1) (8,2,1)
 *     (8,4,1) (16,1,1) (16,2,1) (32,1,1) (32,2,1) (64,1,1) (16,1,4) (32,1,4)
 *     (32,2,4) (64,1,4) (64,2,4) (64,4,4) (32,1,8).
 *   Q4_GEMV_KERNEL_STREAM: one token (n = 1), rows of at most 14560 weights;
 *     each workgroup owns one contiguous range of rows, stages x once and
 *     keeps `depth` weight slots in flight per lane; rows_per_lane is 1.
 *     Instantiated (lanes_per_row, waves_per_group, depth): (8,16,2)
 *     (16,16,2) (16,1,2) (32,1,2) (32,8,2) (32,16,2) (64,4,2) (64,8,2)
 *     (64,16,2) (64,8,3) (64,16,4).
 *   Q4_GEMV_KERNEL_MATRIX: Q4_K only, n = 1..8: the products on matrix cores
 *     (v_mfma_f32_16x16x32_f16 on 16-row tiles); one 8-wave workgroup per
 *     compute unit (times groups_per_cu, the only geometry field it takes;
 *     the others must be 0) owns a contiguous range of tiles and stages x
 *     once (in chunks when the row does not fit the LDS).
 * With kernel Q4_GEMV_KERNEL_AUTO, a tuning that sets any geometry field
 * names a tiled geometry; one that sets none keeps the library's choice of
 * kernel. Other geometries return Q4_EUNSUPPORTED. */
enum { Q4_GEMV_KERNEL_AUTO = 0, Q4_GEMV_KERNEL_TILED = 1, Q4_GEMV_KERNEL_STREAM = 2, Q4_GEMV_KERNEL_MATRIX = 3 };
typedef struct {
    int lanes_per_row;   /* lanes sharing one weight row: 8, 16, 32 or 64 */
    int rows_per_lane;   /* rows each lane streams at once: 1, 2 or 4 (streaming: 1) */
    int waves_per_group; /* waves per workgroup */
    int groups_per_cu;   /* workgroups per compute unit the grid is sized for (0..64) */
    int kernel;          /* Q4_GEMV_KERNEL_* */
    int depth;           /* streaming kernel: weight slots in flight per lane */
} q4_gemv_tuning;

/* q4_gemv with an explicit kernel and geometry; same arguments, layouts,
 * results and errors, plus Q4_EINVAL for a null tuning, a negative field or
 * an unknown kernel, and Q4_EUNSUPPORTED for a geometry that is not
 * instantiated, the streaming kernel at n > 1 or beyond its row length, or
 * the matrix-core kernel on a format other than Q4_K or with a geometry field
 * other than groups_per_cu. */
int q4_gemv_tuned(int fmt, const void *w, const float *x, float *y,
                  int64_t m, int64_t k, int64_t n, const q4_gemv_tuning *tuning, void *hip_stream);

/* q4_gemv_addnorm with an explicit tile geometry; same arguments, results and
 * errors, plus Q4_EINVAL for a null tuning, a negative field or an unknown
 * kernel, and Q4_EUNSUPPORTED for the streaming or matrix-core kernel (a tuned
 * fused product runs on the tiled kernel; the untuned plain form takes the
 * streaming kernel where the plain one-token product does) or a geometry that
 * is not instantiated for the fused product. Instantiated:
 * (8,1,1) (8,2,1) (16,1,1) (16,1,4) (32,1,4) (32,1,8) (32,2,1) (32,2,4) (64,1,4)
 * with Q4_EPILOGUE_NONE; (16,2,1) (16,2,4) (32,2,1) (32,2,4) (32,2,8) (64,2,4)
 * with Q4_EPILOGUE_SILU_MUL. */
int q4_gemv_addnorm_tuned(int fmt, const void *w, const float *x, const float *delta, const float *gain, float eps,
                          float *x_out, float *y, int64_t m, int64_t k, int epilogue,
                          const q4_gemv_tuning *tuning, void *hip_stream);

/* Prefill product Y[t][i] = sum_k bf16_rne(w_hat[i][k]) * X[t][k], fp32 out.
 * w: device, quantized as above (any format), 16-byte aligned; x_bf16: device bf16 bit
 * patterns [n][k], 4-byte aligned; y: device float32 [n][m], 4-byte aligned.
 * n >= 1 (any token count). Weight tiles are dequantized to bf16 into LDS
 * and reused across the token tile by bf16 matrix-core (MFMA) instructions
 * with fp32 accumulation (Methodology section 3: dequantize into shared
 * memory and reuse for the matrix-matrix product). A NaN among token t's
 * activations makes every Y[t][i] NaN; the other tokens are unaffected. */
int q4_gemm(int fmt, const void *w, const uint16_t *x_bf16, float *y,
            int64_t m, int64_t k, int64_t n, void *hip_stream);

/* Tile geometry of the prefill product: tile_rows x tile_tokens outputs per
 * workgroup, stage_k weights per row dequantized into LDS per chunk of K (a
 * zero field keeps the library's choice). Instantiated (rows, tokens,
 * stage_k): (16,64,512) (16,64,1024) (32,64,256) (32,64,512) (32,64,1024)
 * (32,128,512) (64,64,256) (64,64,512); others return Q4_EUNSUPPORTED. */
typedef struct {
    int tile_rows;
    int tile_tokens;
    int stage_k;
} q4_gemm_tuning;

/* q4_gemm with an explicit tile geometry; same arguments, layouts, results
 * and errors, plus Q4_EINVAL for a null or negative tuning. */
int q4_gemm_tuned(int fmt, const void *w, const uint16_t *x_bf16, float *y,
                  int64_t m, int64_t k, int64_t n, const q4_gemm_tuning *tuning, void *hip_stream);

/* Epilogue of a layer-stack product. */
enum {
    Q4_EPILOGUE_NONE = 0,     /* y = W x (q4_gemv); w has m rows */
    Q4_EPILOGUE_SILU_MUL = 1  /* y = silu(W_gate x) * (W_up x) (q4_gemv_glu); w has 2m rows */
};

/* One decode product of a layer stack. */
typedef struct {
    const void *w;   /* device weights */
    const float *x;  /* device [n][k] */
    float *y;        /* device [n][m] */
    int64_t m, k;    /* output rows, input length */
    int epilogue;    /* Q4_EPILOGUE_*; any other value is Q4_EINVAL */
} q4_gemv_op;

/* Enqueue count decode products back-to-back on one stream with no host
 * synchronization in between (the runtime batches kernel submissions and
 * avoids CPU-GPU synchronization: Llamas on the Web, technical summary,
 * Methodology section 2, "execution scheduling"). Every op is validated
 * before the first launch; on error nothing is enqueued. */
int q4_gemv_sequence(int fmt, const q4_gemv_op *ops, int count, int64_t n, void *hip_stream);

/* The same sequence captured once into a HIP graph and replayed with one
 * launch per step (no per-step launch setup: compiled pipelines are cached
 * after the first pass, same section). *graph_out receives a caller-owned
 * handle; the op pointers are baked into the graph. */
typedef struct q4_graph q4_graph;
int q4_graph_create(int fmt, const q4_gemv_op *ops, int count, int64_t n, void *hip_stream,
                    q4_graph **graph_out);
int q4_graph_launch(q4_graph *graph, void *hip_stream);
int q4_graph_destroy(q4_graph *graph);

/* ---- A whole synthetic decode step (Llama family) ----------------------------
 * The decode step of a Llama-family model (the SmolLM2 models the MicroLLM Lab
 * post runs) around the quantized products: the token's embedding (a row of the
 * tied LM-head matrix, dequantized), then per layer
 *   x += delta (from the second layer on); h = rmsnorm(x) * norm_attn;
 *   qkv = W_qkv h (q|k|v stacked); rotary embedding of q and k (rotate-half,
 *   angle pos * theta^(-2i/head_dim)); k and v appended to the caches at pos;
 *   att = grouped-query attention over positions 0..pos (query head h reads
 *   key/value head h / (heads / kv_heads), softmax of q.k / sqrt(head_dim));
 *   delta = W_o att; x += delta; h = rmsnorm(x) * norm_mlp;
 *   act = silu(W_gate h) * (W_up h) (the gated product); delta = W_down act;
 * then x += delta, h = rmsnorm(x) * norm_final, logits = W_emb h, and the next
 * token = argmax(logits) (lowest index among equals), with pos advanced by one.
 * rmsnorm(x) = x / sqrt(mean(x^2) + norm_eps). Keys and values stay cached and
 * the selection runs on the device (WebGPT README, "Roadmap"); all buffers are
 * the caller's (Llamas on the Web, technical summary, Methodology section 1).
 * The token and its position are device int32 values read by the step's
 * kernels, so a captured step replays as a generation loop. A position outside
 * [0, max_pos) makes the attention outputs NaN and writes no cache entry.
 * Each residual add and RMSNorm runs inside the product that consumes it
 * (q4_gemv_addnorm): the residual stream alternates between the buffers x and
 * h (a product reads one and writes x + delta to the other), and after the
 * step h holds the final residual stream x + delta. */
typedef struct {
    int layers, hidden, heads, kv_heads, head_dim, ffn, vocab, max_pos;
    float rope_theta, norm_eps;
} q4_llama_config;

typedef struct {
    const void *qkv;        /* (heads + 2 kv_heads) * head_dim rows x hidden */
    const void *o;          /* hidden rows x heads * head_dim */
    const void *gate_up;    /* 2 ffn rows (gate, then up) x hidden, as for q4_gemv_glu */
    const void *down;       /* hidden rows x ffn */
    const float *norm_attn, *norm_mlp;  /* hidden each, device, 16-byte aligned */
} q4_llama_layer;

typedef struct {            /* device buffers, all caller-owned (16-byte aligned) */
    float *x, *h;           /* hidden each: the residual stream, alternating between the two */
    float *qkv;             /* (heads + 2 kv_heads) * head_dim */
    float *att;             /* heads * head_dim */
    float *delta;           /* hidden */
    float *act;             /* ffn */
    float *logits;          /* vocab */
    float *k_cache, *v_cache;  /* layers x kv_heads x max_pos x head_dim each */
    int32_t *token;         /* [1]: the current token in, the next token out */
    int32_t *pos;           /* [1]: the current token's position, advanced by one */
} q4_llama_state;

/* Enqueue one decode step (fmt for every matrix; emb: vocab x hidden, also the
 * LM head; norm_final: hidden, device, 16-byte aligned). Limits: head_dim 32,
 * 64 or 128; max_pos at most 8192; hidden at most 14560; hidden,
 * heads * head_dim and ffn whole numbers of blocks. Errors as q4_gemv for each product, Q4_EINVAL for a null
 * pointer or an inconsistent configuration, Q4_EUNSUPPORTED beyond the limits. */
int q4_llama_step(int fmt, const q4_llama_config *cfg, const void *emb, const float *norm_final,
                  const q4_llama_layer *layers, const q4_llama_state *state, void *hip_stream);

/* q4_llama_step for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * The same step, kernels and results, except that the intermediate vectors
 * (state->qkv, att, delta, act: ignored here, may be null) live in a static
 * device array of the library: 65536 floats (256 KiB) per GPU, held until the
 * process ends. Each vector takes its length rounded up to a multiple of 16
 * floats; a configuration needing more than 65536 in total
 * ((heads + 2 kv_heads) * head_dim + heads * head_dim + hidden + ffn, so
 * rounded) returns Q4_EUNSUPPORTED with nothing enqueued. Other arguments and
 * errors as q4_llama_step. Calls no allocating routine; the array's address is
 * looked up on the first call on each device (Q4_EHIP if that fails), so a
 * caller that captures the call into a HIP graph makes one call on that
 * device outside capture first. The
 * array keeps the last call's contents and nothing in it must start at zero
 * (every vector is written before it is read within a step). Every call on one
 * GPU shares that GPU's array: calls that overlap on one GPU (on different
 * streams, or a graph that captured this call replayed beside another) race. */
int q4_llama_step_noalloc(int fmt, const q4_llama_config *cfg, const void *emb, const float *norm_final,
                          const q4_llama_layer *layers, const q4_llama_state *state, void *hip_stream);

/* The same step captured once into a HIP graph; each launch runs one step. */
typedef struct q4_llama_graph q4_llama_graph;
int q4_llama_graph_create(int fmt, const q4_llama_config *cfg, const void *emb, const float *norm_final,
                          const q4_llama_layer *layers, const q4_llama_state *state, void *hip_stream,
                          q4_llama_graph **graph_out);
int q4_llama_graph_launch(q4_llama_graph *graph, void *hip_stream);
int q4_llama_graph_destroy(q4_llama_graph *graph);

/* Static string for a status code (the C ABI's own error reporting, not a
 * step of the method, so no passage defines it; an unknown code gets a
 * generic string). */
const char *q4_strerror(int status);

/* Name of the HIP error behind the calling thread's most recent Q4_EHIP
 * ("hipSuccess" if there was none); a static string. */
const char *q4_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* Q4_H */
