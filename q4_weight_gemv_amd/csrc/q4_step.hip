// A whole synthetic decode step of a Llama-family model around the quantized
// matrix products (the SmolLM2 models of the MicroLLM Lab post, "Seven models,
// all in Q4"): embedding, per layer a residual add with RMSNorm, the stacked
// q|k|v product, rotary embedding, KV-cache append and grouped-query attention,
// the output projection, a second add with RMSNorm, the gated MLP and the down
// projection; the final norm, the tied LM head and the greedy token. Keys and
// values stay cached between steps and the token selection runs on the device
// (WebGPT README, "Roadmap"); every buffer is the caller's, allocated up front
// (Llamas on the Web, technical summary, Methodology section 1).
//
// The products are the library's decode kernels (q4_gemv, and for the
// products that follow a norm the fused residual add + RMSNorm variant,
// q4_gemv_addnorm); the kernels here are the small operators between them:
// the embedding gather, attention and the token selection. The token and its
// position live in device memory, read by the kernels and advanced by the last
// one, so a captured step replays as a generation loop with no host work.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <new>

#include "q4_internal.h"

namespace q4 {
namespace step {

constexpr int kThreads = 256;
constexpr int kMaxPos = 8192;       // scores of one head live in LDS

__device__ __forceinline__ float block_sum(float v, float *red)
{
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    __syncthreads();  // red may still be read by a previous reduction
    if (lane == 0) red[wave] = v;
    __syncthreads();
    float s = 0.0f;
    for (int i = 0; i < kThreads / 64; i++) s += red[i];
    return s;
}

__device__ __forceinline__ float block_max(float v, float *red)
{
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    __syncthreads();
    if (lane == 0) red[wave] = v;
    __syncthreads();
    float s = red[0];
    for (int i = 1; i < kThreads / 64; i++) s = fmaxf(s, red[i]);
    return s;
}

// Sum over W consecutive lanes (W = 8, 16 or 32, groups aligned to W), by
// exchanges in a butterfly: every lane of the group ends with the same total.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

template <int W>
__device__ __forceinline__ float lane_group_sum(float v)
{
    static_assert(W == 8 || W == 16 || W == 32, "lane group of 8, 16 or 32");
    v += dpp_f<0xB1>(v);   // quad_perm [1,0,3,2]: lane ^ 1
    v += dpp_f<0x4E>(v);   // quad_perm [2,3,0,1]: lane ^ 2
    v += dpp_f<0x141>(v);  // row_half_mirror: lane 7 - i of its 8 (the other quad)
    if constexpr (W >= 16) v += dpp_f<0x140>(v);  // row_mirror: lane 15 - i of its 16 (the other 8)
    if constexpr (W >= 32) v += __shfl_xor(v, 16);
    return v;
}

// Dequantized weight (r, c) of a quantized m x k matrix, any format (one value;
// the embedding gather reads one row).
__device__ float weight_at(int fmt, const uint8_t *w, int64_t m, int64_t k, int64_t r, int64_t c)
{
    auto half = [](const uint8_t *p) { return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(p[0] | (p[1] << 8)))); };
    if (fmt == Q4_FMT_Q4_0) {
        const int64_t b = r * (k / 32) + c / 32, e = c % 32;
        const uint8_t byte = w[b * 16 + (e & 15)];
        const int q = e < 16 ? (byte & 15) : (byte >> 4);
        return static_cast<float>(q - 8) * half(w + m * k / 2 + b * 2);
    }
    if (fmt == Q4_FMT_Q8_0) {
        const int64_t b = r * (k / 32) + c / 32;
        return static_cast<float>(static_cast<int8_t>(w[b * 32 + c % 32])) * half(w + m * k + b * 2);
    }
    if (fmt == Q4_FMT_Q1_0) {
        const int64_t b = r * (k / 32) + c / 32;
        const int e = static_cast<int>(c % 32);
        const float d = half(w + m * k / 8 + b * 2);
        return (w[b * 4 + e / 8] >> (e % 8)) & 1 ? d : -d;
    }
    const int64_t s = r * (k / 256) + c / 256;
    const int e = static_cast<int>(c % 256);
    if (fmt == Q4_FMT_Q2_K) {
        const int q = (w[s * 64 + 32 * (e / 128) + e % 32] >> (2 * ((e % 128) / 32))) & 3;
        const uint8_t sm = w[m * k / 4 + s * 16 + e / 16];
        const uint8_t *dd = w + m * k * 5 / 16 + s * 4;
        return (half(dd) * static_cast<float>(sm & 15)) * static_cast<float>(q) - half(dd + 2) * static_cast<float>(sm >> 4);
    }
    // Q4_K
    const uint8_t *sb = w + s * 144;
    const int j = e / 32;
    const uint8_t byte = sb[16 + 32 * (e / 64) + e % 32];
    const int q = (e % 64) >= 32 ? (byte >> 4) : (byte & 15);
    const uint8_t *S = sb + 4;
    const int sc = j < 4 ? (S[j] & 63) : ((S[j + 4] & 15) | ((S[j - 4] >> 6) << 4));
    const int mn = j < 4 ? (S[j + 4] & 63) : ((S[j + 4] >> 4) | ((S[j] >> 6) << 4));
    return (half(sb) * static_cast<float>(sc)) * static_cast<float>(q) - half(sb + 2) * static_cast<float>(mn);
}

// x = row `token` of the embedding matrix (the tied LM head), dequantized.
__global__ __launch_bounds__(kThreads) void embed_kernel(int fmt, const uint8_t *__restrict__ emb, int vocab, int hidden,
                                                         const int32_t *__restrict__ token, float *__restrict__ x)
{
    int t = token[0];
    if (t < 0 || t >= vocab) t = 0;  // never read outside the matrix
    for (int i = threadIdx.x; i < hidden; i += kThreads) x[i] = weight_at(fmt, emb, vocab, hidden, t, i);
}

// Rotary angle of pair i of a head of dim d at position pos.
__device__ __forceinline__ void rope_cs(int i, int d, int pos, float log2_theta, float &c, float &s)
{
    const float inv = exp2f(-2.0f * static_cast<float>(i) / static_cast<float>(d) * log2_theta);
    sincosf(static_cast<float>(pos) * inv, &s, &c);
}

// Grouped-query attention for one query head per workgroup, at the position
// held in pos[0]: rotates the head's query and its key/value head's new key,
// appends key and value to the caches (the group's first head writes them),
// then softmax(q . k_t / sqrt(D)) over t <= pos and the weighted sum of values.
// Caches: [kv_heads][max_pos][D]. A position outside [0, max_pos) writes NaN
// outputs and touches no cache.
// The step's q, k and v are loaded alongside the position. Keys and values
// are read alike: thread (c, r) holds dimensions 4c..4c+3 of positions r,
// r + RR, ... (RR = 256 / (D/4)), so each load instruction of a wave reads
// whole rows, contiguous in the cache; VJ rows per thread are loaded at once
// (rows past pos read row pos and are dropped; the current position's key
// and value come from LDS, since another workgroup may be writing them to
// the cache). A score is the sum of its row's D/4 partial dot products,
// formed across those lanes by a butterfly. The first VJ value rows are
// loaded with the first key rows so that their latency overlaps the scores
// and the softmax; the per-thread sums of weighted values meet in LDS at the
// end.
template <int D>
__global__ __launch_bounds__(kThreads) void attention_kernel(const float *__restrict__ qkv, float *__restrict__ kcache,
                                                             float *__restrict__ vcache, const int32_t *__restrict__ posp,
                                                             int heads, int kv_heads, int max_pos, float log2_theta,
                                                             float *__restrict__ out)
{
    typedef float f4 __attribute__((ext_vector_type(4)));
    constexpr int VQ = D / 4;          // 16-byte pieces per row
    constexpr int RR = kThreads / VQ;  // value rows per round of the workgroup
    constexpr int VJ = 16;             // value rows per thread per chunk
    constexpr int CH = RR * VJ;        // positions per value chunk
    __shared__ __attribute__((aligned(16))) float qs[D];
    __shared__ __attribute__((aligned(16))) float ks[D];
    __shared__ __attribute__((aligned(16))) float vs[D];
    __shared__ float scores[kMaxPos];
    __shared__ __attribute__((aligned(16))) float part[RR * D];
    __shared__ float red[kThreads / 64];
    constexpr int half = D / 2;
    const int h = blockIdx.x;
    const int g = h / (heads / kv_heads);
    const int tid = threadIdx.x;
    const float *q = qkv + h * D;
    const float *k = qkv + heads * D + g * D;
    const float *v = qkv + (heads + kv_heads) * D + g * D;
    float q0 = 0.0f, q1 = 0.0f, k0 = 0.0f, k1 = 0.0f, v0 = 0.0f;
    if (tid < half) {
        q0 = q[tid];
        q1 = q[tid + half];
        k0 = k[tid];
        k1 = k[tid + half];
    }
    if (tid < D) v0 = v[tid];
    const int pos = posp[0];
    if (pos < 0 || pos >= max_pos) {
        for (int i = tid; i < D; i += kThreads) out[h * D + i] = __builtin_nanf("");
        return;
    }
    if (tid < half) {
        float c, s;
        rope_cs(tid, D, pos, log2_theta, c, s);
        qs[tid] = q0 * c - q1 * s;
        qs[tid + half] = q1 * c + q0 * s;
        ks[tid] = k0 * c - k1 * s;
        ks[tid + half] = k1 * c + k0 * s;
    }
    if (tid < D) vs[tid] = v0;
    __syncthreads();
    float *kc = kcache + static_cast<size_t>(g) * max_pos * D;
    float *vc = vcache + static_cast<size_t>(g) * max_pos * D;
    if (h % (heads / kv_heads) == 0 && tid < D) {
        kc[static_cast<size_t>(pos) * D + tid] = ks[tid];
        vc[static_cast<size_t>(pos) * D + tid] = vs[tid];
    }
    const float scale = 1.0f / sqrtf(static_cast<float>(D));
    const int vcol = tid % VQ, vrow0 = tid / VQ;
    // This thread's four dimensions of the query and of the current key.
    const f4 qq = reinterpret_cast<const f4 *>(qs)[vcol];
    const f4 kcur = reinterpret_cast<const f4 *>(ks)[vcol];
    // Rows t0 + vrow0 + j*RR (j < VJ) of a cache, dimensions 4*vcol..+3.
    auto cache_rows = [&](const float *cache, int t0, f4(&r)[VJ]) {
#pragma unroll
        for (int j = 0; j < VJ; j++) {
            const int t = t0 + vrow0 + j * RR;
            r[j] = reinterpret_cast<const f4 *>(cache + static_cast<size_t>(t < pos ? t : pos) * D)[vcol];
        }
    };
    float mx = -INFINITY;
    auto score_rows = [&](int t0, const f4(&r)[VJ]) {
#pragma unroll
        for (int j = 0; j < VJ; j++) {
            if (t0 + j * RR > pos) break;  // the slice's rows all lie past pos (uniform)
            const int t = t0 + vrow0 + j * RR;
            const f4 kk = t == pos ? kcur : r[j];
            float p = qq.x * kk.x;
            p = fmaf(qq.y, kk.y, p);
            p = fmaf(qq.z, kk.z, p);
            p = fmaf(qq.w, kk.w, p);
            const float sc = lane_group_sum<VQ>(p) * scale;  // every lane of the row
            if (t <= pos) {
                if (vcol == 0) scores[t] = sc;
                mx = fmaxf(mx, sc);
            }
        }
    };
    f4 vrows[VJ];
    {
        f4 kr[VJ];
        cache_rows(kc, 0, kr);
        cache_rows(vc, 0, vrows);
        score_rows(0, kr);
    }
    for (int t0 = CH; t0 <= pos; t0 += CH) {
        f4 kr[VJ];
        cache_rows(kc, t0, kr);
        score_rows(t0, kr);
    }
    mx = block_max(mx, red);
    float sum = 0.0f;
    for (int t = tid; t <= pos; t += kThreads) {
        const float e = expf(scores[t] - mx);
        scores[t] = e;
        sum += e;
    }
    sum = block_sum(sum, red);  // its barriers also publish scores[]
    const f4 vcur = reinterpret_cast<const f4 *>(vs)[vcol];
    f4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    auto accumulate = [&](int t0) {
#pragma unroll
        for (int j = 0; j < VJ; j++) {
            if (t0 + j * RR > pos) break;  // the slice's rows all lie past pos (uniform)
            const int t = t0 + vrow0 + j * RR;
            const float w = scores[t < pos ? t : pos];
            const f4 vv = t == pos ? vcur : vrows[j];
            const f4 a = acc + w * vv;
            acc = t <= pos ? a : acc;
        }
    };
    accumulate(0);
    for (int t0 = CH; t0 <= pos; t0 += CH) {
        cache_rows(vc, t0, vrows);
        accumulate(t0);
    }
    reinterpret_cast<f4 *>(part)[vrow0 * VQ + vcol] = acc;
    __syncthreads();
    if (tid < D) {
        float o = 0.0f;
#pragma unroll
        for (int r = 0; r < RR; r++) o += part[r * D + tid];
        out[h * D + tid] = o / sum;
    }
}

// Greedy selection: token[0] = the index of the largest logit (the lowest
// index among equals; NaN logits never win), then pos[0] += 1.
__global__ __launch_bounds__(1024) void argmax_advance_kernel(const float *__restrict__ logits, int n,
                                                              int32_t *__restrict__ token, int32_t *__restrict__ pos)
{
    __shared__ float bv[16];
    __shared__ int bi[16];
    float best = -INFINITY;
    int idx = 0x7FFFFFFF;
#pragma unroll 8
    for (int i = threadIdx.x; i < n; i += 1024) {  // indices ascend, so a strict > keeps the lowest
        const float v = logits[i];
        if (v > best) {
            best = v;
            idx = i;
        }
    }
    for (int o = 32; o > 0; o >>= 1) {
        const float ov = __shfl_xor(best, o);
        const int oi = __shfl_xor(idx, o);
        if (ov > best || (ov == best && oi < idx)) {
            best = ov;
            idx = oi;
        }
    }
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    if (lane == 0) {
        bv[wave] = best;
        bi[wave] = idx;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 1; w < 16; w++)
            if (bv[w] > best || (bv[w] == best && bi[w] < idx)) {
                best = bv[w];
                idx = bi[w];
            }
        token[0] = idx == 0x7FFFFFFF ? 0 : idx;
        pos[0] = pos[0] + 1;
    }
}

}  // namespace step
}  // namespace q4

namespace {

bool multiple(int64_t v, int64_t b) { return v > 0 && v % b == 0; }

int check_step(int fmt, const q4_llama_config *c, const void *emb, const float *norm_final, const q4_llama_layer *L,
               const q4_llama_state *st)
{
    using namespace q4::step;
    if (!c || !emb || !norm_final || !L || !st) return Q4_EINVAL;
    if (fmt != Q4_FMT_Q4_0 && fmt != Q4_FMT_Q4_K && fmt != Q4_FMT_Q8_0 && fmt != Q4_FMT_Q2_K && fmt != Q4_FMT_Q1_0)
        return Q4_EUNSUPPORTED;
    const int64_t blk = fmt == Q4_FMT_Q4_K || fmt == Q4_FMT_Q2_K ? 256 : 32;
    if (c->layers <= 0 || c->heads <= 0 || c->kv_heads <= 0 || c->heads % c->kv_heads || c->vocab <= 0 ||
        c->max_pos <= 0 || !(c->norm_eps >= 0.0f) || !(c->rope_theta > 0.0f))
        return Q4_EINVAL;
    if (c->head_dim != 32 && c->head_dim != 64 && c->head_dim != 128) return Q4_EUNSUPPORTED;
    if (c->max_pos > kMaxPos || c->hidden > q4::kNormMaxUnits * q4::kUnitWeights) return Q4_EUNSUPPORTED;
    // Every product's input length is a whole number of blocks.
    if (!multiple(c->hidden, blk) || !multiple(static_cast<int64_t>(c->heads) * c->head_dim, blk) || !multiple(c->ffn, blk))
        return Q4_EINVAL;
    if (!st->x || !st->h || !st->qkv || !st->att || !st->delta || !st->act || !st->logits || !st->k_cache ||
        !st->v_cache || !st->token || !st->pos)
        return Q4_EINVAL;
    // The attention reads cache rows as 16-byte vectors.
    if ((reinterpret_cast<uintptr_t>(st->k_cache) & 15) || (reinterpret_cast<uintptr_t>(st->v_cache) & 15))
        return Q4_EALIGN;
    const int64_t qkv_n = static_cast<int64_t>(c->heads + 2 * c->kv_heads) * c->head_dim;
    const int64_t hd = c->hidden, qn = static_cast<int64_t>(c->heads) * c->head_dim;
    // The residual stream alternates between x and h; each fused-norm product
    // reads one and the delta and writes the other.
    auto norm_io = [&](const float *gain, float *out) {
        q4::Prologue p;
        p.delta = st->delta;
        p.gain = gain;
        p.x_out = out;
        p.eps = c->norm_eps;
        return p;
    };
    for (int i = 0; i < c->layers; i++) {
        if (!L[i].norm_attn || !L[i].norm_mlp) return Q4_EINVAL;
        int s = q4::check_addnorm_args(fmt, L[i].qkv, st->x, norm_io(L[i].norm_attn, st->h), st->qkv, qkv_n, hd, false);
        if (s == Q4_OK) s = q4::check_product_args(fmt, L[i].o, st->att, st->delta, hd, qn, 1, 8);
        if (s == Q4_OK)
            s = q4::check_addnorm_args(fmt, L[i].gate_up, st->h, norm_io(L[i].norm_mlp, st->x), st->act, c->ffn, hd, true);
        if (s == Q4_OK) s = q4::check_product_args(fmt, L[i].down, st->act, st->delta, hd, c->ffn, 1, 8);
        if (s != Q4_OK) return s;
    }
    return q4::check_addnorm_args(fmt, emb, st->x, norm_io(norm_final, st->h), st->logits, c->vocab, hd, false);
}

int enqueue_step(int fmt, const q4_llama_config *c, const void *emb, const float *norm_final, const q4_llama_layer *L,
                 const q4_llama_state *st, hipStream_t s)
{
    using namespace q4::step;
    const int64_t hd = c->hidden, qn = static_cast<int64_t>(c->heads) * c->head_dim;
    const int64_t qkv_n = qn + 2LL * c->kv_heads * c->head_dim;
    const size_t cache_layer = static_cast<size_t>(c->kv_heads) * c->max_pos * c->head_dim;
    const float log2_theta = std::log2(c->rope_theta);
    auto ok = [](hipError_t e) { return q4::hip_status(e); };
    // Residual add + RMSNorm fused into the next product: it reads the stream
    // from `in` (plus delta) and writes the updated stream to `out`.
    auto addnorm = [&](const void *w, const float *in, bool add, const float *gain, float *out, float *y, int64_t m,
                       bool glu) {
        q4::Prologue p;
        p.delta = add ? st->delta : nullptr;
        p.gain = gain;
        p.x_out = out;
        p.eps = c->norm_eps;
        return q4::launch_gemv_addnorm(fmt, w, in, p, y, m, hd, glu, s);
    };
    hipLaunchKernelGGL(embed_kernel, dim3(1), dim3(kThreads), 0, s, fmt, static_cast<const uint8_t *>(emb), c->vocab,
                       c->hidden, st->token, st->x);
    int r = ok(hipGetLastError());
    for (int i = 0; i < c->layers && r == Q4_OK; i++) {
        // x (+ the previous layer's delta) -> h.
        r = addnorm(L[i].qkv, st->x, i > 0, L[i].norm_attn, st->h, st->qkv, qkv_n, false);
        if (r == Q4_OK) {
            float *kc = st->k_cache + i * cache_layer, *vc = st->v_cache + i * cache_layer;
            if (c->head_dim == 32)
                hipLaunchKernelGGL(attention_kernel<32>, dim3(c->heads), dim3(kThreads), 0, s, st->qkv, kc, vc, st->pos,
                                   c->heads, c->kv_heads, c->max_pos, log2_theta, st->att);
            else if (c->head_dim == 64)
                hipLaunchKernelGGL(attention_kernel<64>, dim3(c->heads), dim3(kThreads), 0, s, st->qkv, kc, vc, st->pos,
                                   c->heads, c->kv_heads, c->max_pos, log2_theta, st->att);
            else
                hipLaunchKernelGGL(attention_kernel<128>, dim3(c->heads), dim3(kThreads), 0, s, st->qkv, kc, vc, st->pos,
                                   c->heads, c->kv_heads, c->max_pos, log2_theta, st->att);
            r = ok(hipGetLastError());
        }
        if (r == Q4_OK) r = q4::launch_gemv(fmt, L[i].o, st->att, st->delta, hd, qn, 1, s);
        // h + delta -> x.
        if (r == Q4_OK) r = addnorm(L[i].gate_up, st->h, true, L[i].norm_mlp, st->x, st->act, c->ffn, true);
        if (r == Q4_OK) r = q4::launch_gemv(fmt, L[i].down, st->act, st->delta, hd, c->ffn, 1, s);
    }
    if (r != Q4_OK) return r;
    // x + delta -> h: the final stream.
    r = addnorm(emb, st->x, true, norm_final, st->h, st->logits, c->vocab, false);
    if (r == Q4_OK) {
        hipLaunchKernelGGL(argmax_advance_kernel, dim3(1), dim3(1024), 0, s, st->logits, c->vocab, st->token, st->pos);
        r = ok(hipGetLastError());
    }
    return r;
}

}  // namespace

struct q4_llama_graph {
    hipGraph_t graph = nullptr;
    hipGraphExec_t exec = nullptr;
};

// Workspace of q4_llama_step_noalloc: the step's intermediate vectors (q|k|v,
// attention output, delta, gated activation) in a file-scope device array.
// Each GPU holds its own copy until the process ends; host code reaches it
// only through the device address that hipGetSymbolAddress returns for the
// current device (the array's name on the host is not a device address).
constexpr int64_t kStepScratchFloats = 65536;  // 256 KiB per GPU
static __device__ __align__(256) float scratch[kStepScratchFloats];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<float *> scratch_dev[kMaxDevices];

// The current device's copy of `scratch`, looked up on the first call on
// that device (with it current) and kept.
int step_scratch(float **out)
{
    int dev = 0;
    int st = q4::hip_status(hipGetDevice(&dev));
    if (st != Q4_OK) return st;
    if (dev < 0 || dev >= kMaxDevices) return Q4_EUNSUPPORTED;
    float *p = scratch_dev[dev].load(std::memory_order_acquire);
    if (!p) {
        void *a = nullptr;
        st = q4::hip_status(hipGetSymbolAddress(&a, HIP_SYMBOL(scratch)));
        if (st != Q4_OK) return st;
        if (!a) return Q4_EHIP;
        p = static_cast<float *>(a);
        scratch_dev[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return Q4_OK;
}

int64_t round16(int64_t n) { return n > 0 ? (n + 15) / 16 * 16 : 0; }

}  // namespace

extern "C" {

int q4_llama_step(int fmt, const q4_llama_config *cfg, const void *emb, const float *norm_final,
                  const q4_llama_layer *layers, const q4_llama_state *state, void *hip_stream)
{
    const int st = check_step(fmt, cfg, emb, norm_final, layers, state);
    if (st != Q4_OK) return st;
    return enqueue_step(fmt, cfg, emb, norm_final, layers, state, static_cast<hipStream_t>(hip_stream));
}

int q4_llama_graph_create(int fmt, const q4_llama_config *cfg, const void *emb, const float *norm_final,
                          const q4_llama_layer *layers, const q4_llama_state *state, void *hip_stream,
                          q4_llama_graph **graph_out)
{
    if (!graph_out) return Q4_EINVAL;
    *graph_out = nullptr;
    int st = check_step(fmt, cfg, emb, norm_final, layers, state);
    if (st != Q4_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    hipStream_t own = nullptr;
    if (!s) {
        st = q4::hip_status(hipStreamCreateWithFlags(&own, hipStreamNonBlocking));
        if (st != Q4_OK) return st;
        s = own;
    }
    auto *g = new (std::nothrow) q4_llama_graph();
    if (!g) {
        if (own) (void)hipStreamDestroy(own);
        return Q4_EHIP;
    }
    st = q4::hip_status(hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal));
    if (st == Q4_OK) {
        const int est = enqueue_step(fmt, cfg, emb, norm_final, layers, state, s);
        const int end = q4::hip_status(hipStreamEndCapture(s, &g->graph));
        st = est != Q4_OK ? est : end;
    }
    if (st == Q4_OK) st = q4::hip_status(hipGraphInstantiate(&g->exec, g->graph, nullptr, nullptr, 0));
    if (own) (void)hipStreamDestroy(own);
    if (st != Q4_OK) {
        if (g->exec) (void)hipGraphExecDestroy(g->exec);
        if (g->graph) (void)hipGraphDestroy(g->graph);
        delete g;
        return st;
    }
    *graph_out = g;
    return Q4_OK;
}

int q4_llama_step_noalloc(int fmt, const q4_llama_config *cfg, const void *emb, const float *norm_final,
                          const q4_llama_layer *layers, const q4_llama_state *state, void *hip_stream)
{
    if (!cfg || !state) return Q4_EINVAL;
    // Each vector starts on a 64-byte boundary of the array.
    const int64_t qn = static_cast<int64_t>(cfg->heads) * cfg->head_dim;
    const int64_t qkv_n = (static_cast<int64_t>(cfg->heads) + 2LL * cfg->kv_heads) * cfg->head_dim;
    const int64_t o_att = round16(qkv_n), o_delta = o_att + round16(qn), o_act = o_delta + round16(cfg->hidden);
    const int64_t need = o_act + round16(cfg->ffn);
    const bool fits = need <= kStepScratchFloats;
    // Every argument is validated before any HIP call: the workspace
    // pointers are checked at their offsets from a stand-in base with the
    // array's alignment (checking reads no memory), then rebased onto the
    // device's copy of the array.
    auto place = [&](q4_llama_state &ws, float *base) {
        ws.qkv = base;
        ws.att = base + (fits ? o_att : 0);
        ws.delta = base + (fits ? o_delta : 0);
        ws.act = base + (fits ? o_act : 0);
    };
    q4_llama_state ws = *state;
    place(ws, reinterpret_cast<float *>(static_cast<uintptr_t>(256)));
    int st = check_step(fmt, cfg, emb, norm_final, layers, &ws);
    if (st != Q4_OK) return st;
    if (!fits) return Q4_EUNSUPPORTED;
    float *base = nullptr;
    st = step_scratch(&base);
    if (st != Q4_OK) return st;
    place(ws, base);
    return enqueue_step(fmt, cfg, emb, norm_final, layers, &ws, static_cast<hipStream_t>(hip_stream));
}

int q4_llama_graph_launch(q4_llama_graph *graph, void *hip_stream)
{
    if (!graph || !graph->exec) return Q4_EINVAL;
    return q4::hip_status(hipGraphLaunch(graph->exec, static_cast<hipStream_t>(hip_stream)));
}

int q4_llama_graph_destroy(q4_llama_graph *graph)
{
    if (!graph) return Q4_OK;
    int st = Q4_OK;
    if (graph->exec && hipGraphExecDestroy(graph->exec) != hipSuccess) st = Q4_EHIP;
    if (graph->graph && hipGraphDestroy(graph->graph) != hipSuccess) st = Q4_EHIP;
    delete graph;
    return st;
}

}  // extern "C"
