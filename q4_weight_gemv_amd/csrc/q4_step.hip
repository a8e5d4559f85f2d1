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
// The products are the library's decode kernels (q4_gemv, the gated product);
// the kernels here are the small operators between them. The token and its
// position live in device memory, read by the kernels and advanced by the last
// one, so a captured step replays as a generation loop with no host work.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <new>

#include "q4_internal.h"

namespace q4 {
namespace step {

constexpr int kThreads = 256;
constexpr int kMaxPos = 8192;       // scores of one head live in LDS
constexpr int kMaxHidden = 1 << 20;

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

// x += delta (when given), then h = x / sqrt(mean(x^2) + eps) * g. One group;
// each thread reads its elements in one batch of loads per pass (the loops run
// over ceil(n / 256) elements; the second pass rereads x, this thread's own
// writes of the first).
__global__ __launch_bounds__(kThreads) void add_rmsnorm_kernel(float *__restrict__ x, const float *__restrict__ delta,
                                                               const float *__restrict__ g, float *__restrict__ h,
                                                               int n, float eps)
{
    __shared__ float red[kThreads / 64];
    float ss = 0.0f;
    if (delta) {
#pragma unroll 4
        for (int i = threadIdx.x; i < n; i += kThreads) {
            const float a = x[i] + delta[i];
            x[i] = a;
            ss = fmaf(a, a, ss);
        }
    } else {
#pragma unroll 4
        for (int i = threadIdx.x; i < n; i += kThreads) {
            const float a = x[i];
            ss = fmaf(a, a, ss);
        }
    }
    const float inv = 1.0f / sqrtf(block_sum(ss, red) / static_cast<float>(n) + eps);
#pragma unroll 4
    for (int i = threadIdx.x; i < n; i += kThreads) h[i] = x[i] * inv * g[i];
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
// outputs and touches no cache. Scores: one position per thread, its key row
// read as D/4 16-byte loads issued together; values: thread (i, p) sums
// dimension i over positions p, p + 256/D, ... four at a time.
template <int D>
__global__ __launch_bounds__(kThreads) void attention_kernel(const float *__restrict__ qkv, float *__restrict__ kcache,
                                                             float *__restrict__ vcache, const int32_t *__restrict__ posp,
                                                             int heads, int kv_heads, int max_pos, float log2_theta,
                                                             float *__restrict__ out)
{
    typedef float f4 __attribute__((ext_vector_type(4)));
    __shared__ __attribute__((aligned(16))) float qs[D];
    __shared__ __attribute__((aligned(16))) float ks[D];
    __shared__ float vs[D];
    __shared__ float scores[kMaxPos];
    __shared__ float part[kThreads];
    __shared__ float red[kThreads / 64];
    constexpr int half = D / 2;
    const int h = blockIdx.x;
    const int g = h / (heads / kv_heads);
    const int tid = threadIdx.x;
    const int pos = posp[0];
    if (pos < 0 || pos >= max_pos) {
        for (int i = tid; i < D; i += kThreads) out[h * D + i] = __builtin_nanf("");
        return;
    }
    const float *q = qkv + h * D;
    const float *k = qkv + heads * D + g * D;
    const float *v = qkv + (heads + kv_heads) * D + g * D;
    if (tid < half) {
        float c, s;
        rope_cs(tid, D, pos, log2_theta, c, s);
        qs[tid] = q[tid] * c - q[tid + half] * s;
        qs[tid + half] = q[tid + half] * c + q[tid] * s;
        ks[tid] = k[tid] * c - k[tid + half] * s;
        ks[tid + half] = k[tid + half] * c + k[tid] * s;
    }
    if (tid < D) vs[tid] = v[tid];
    __syncthreads();
    float *kc = kcache + static_cast<size_t>(g) * max_pos * D;
    float *vc = vcache + static_cast<size_t>(g) * max_pos * D;
    if (h % (heads / kv_heads) == 0 && tid < D) {
        kc[static_cast<size_t>(pos) * D + tid] = ks[tid];
        vc[static_cast<size_t>(pos) * D + tid] = vs[tid];
    }
    const float scale = 1.0f / sqrtf(static_cast<float>(D));
    float mx = -INFINITY;
    for (int t = tid; t <= pos; t += kThreads) {
        const f4 *kt = reinterpret_cast<const f4 *>(t == pos ? ks : kc + static_cast<size_t>(t) * D);
        const f4 *qv = reinterpret_cast<const f4 *>(qs);
        f4 r[D / 4];
#pragma unroll
        for (int j = 0; j < D / 4; j++) r[j] = kt[j];
        float s = 0.0f;
#pragma unroll
        for (int j = 0; j < D / 4; j++) {
            const f4 qq = qv[j];
            s = fmaf(qq.x, r[j].x, s);
            s = fmaf(qq.y, r[j].y, s);
            s = fmaf(qq.z, r[j].z, s);
            s = fmaf(qq.w, r[j].w, s);
        }
        s *= scale;
        scores[t] = s;
        mx = fmaxf(mx, s);
    }
    mx = block_max(mx, red);
    float sum = 0.0f;
    for (int t = tid; t <= pos; t += kThreads) {
        const float e = expf(scores[t] - mx);
        scores[t] = e;
        sum += e;
    }
    sum = block_sum(sum, red);  // its barriers also publish scores[]
    constexpr int P = kThreads / D;
    const int i = tid % D, p0 = tid / D;
    float a0 = 0.0f, a1 = 0.0f, a2 = 0.0f, a3 = 0.0f;
    int t = p0;
    for (; t + 3 * P < pos; t += 4 * P) {  // four positions before pos at a time
        const float v0 = vc[static_cast<size_t>(t) * D + i], v1 = vc[static_cast<size_t>(t + P) * D + i];
        const float v2 = vc[static_cast<size_t>(t + 2 * P) * D + i], v3 = vc[static_cast<size_t>(t + 3 * P) * D + i];
        a0 = fmaf(scores[t], v0, a0);
        a1 = fmaf(scores[t + P], v1, a1);
        a2 = fmaf(scores[t + 2 * P], v2, a2);
        a3 = fmaf(scores[t + 3 * P], v3, a3);
    }
    for (; t <= pos; t += P) a0 = fmaf(scores[t], t == pos ? vs[i] : vc[static_cast<size_t>(t) * D + i], a0);
    part[tid] = (a0 + a1) + (a2 + a3);
    __syncthreads();
    if (tid < D) {
        float o = 0.0f;
#pragma unroll
        for (int p = 0; p < P; p++) o += part[p * D + tid];
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
    if (fmt != Q4_FMT_Q4_0 && fmt != Q4_FMT_Q4_K && fmt != Q4_FMT_Q8_0 && fmt != Q4_FMT_Q2_K) return Q4_EUNSUPPORTED;
    const int64_t blk = fmt == Q4_FMT_Q4_K || fmt == Q4_FMT_Q2_K ? 256 : 32;
    if (c->layers <= 0 || c->heads <= 0 || c->kv_heads <= 0 || c->heads % c->kv_heads || c->vocab <= 0 ||
        c->max_pos <= 0 || !(c->norm_eps >= 0.0f) || !(c->rope_theta > 0.0f))
        return Q4_EINVAL;
    if (c->head_dim != 32 && c->head_dim != 64 && c->head_dim != 128) return Q4_EUNSUPPORTED;
    if (c->max_pos > kMaxPos || c->hidden > kMaxHidden) return Q4_EUNSUPPORTED;
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
    for (int i = 0; i < c->layers; i++) {
        if (!L[i].norm_attn || !L[i].norm_mlp) return Q4_EINVAL;
        int s = q4::check_product_args(fmt, L[i].qkv, st->h, st->qkv, qkv_n, hd, 1, 8);
        if (s == Q4_OK) s = q4::check_product_args(fmt, L[i].o, st->att, st->delta, hd, qn, 1, 8);
        if (s == Q4_OK) s = q4::check_glu_args(fmt, L[i].gate_up, st->h, st->act, c->ffn, hd, 1);
        if (s == Q4_OK) s = q4::check_product_args(fmt, L[i].down, st->act, st->delta, hd, c->ffn, 1, 8);
        if (s != Q4_OK) return s;
    }
    return q4::check_product_args(fmt, emb, st->h, st->logits, c->vocab, hd, 1, 8);
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
    hipLaunchKernelGGL(embed_kernel, dim3(1), dim3(kThreads), 0, s, fmt, static_cast<const uint8_t *>(emb), c->vocab,
                       c->hidden, st->token, st->x);
    int r = ok(hipGetLastError());
    for (int i = 0; i < c->layers && r == Q4_OK; i++) {
        hipLaunchKernelGGL(add_rmsnorm_kernel, dim3(1), dim3(kThreads), 0, s, st->x, i == 0 ? nullptr : st->delta,
                           L[i].norm_attn, st->h, c->hidden, c->norm_eps);
        r = ok(hipGetLastError());
        if (r == Q4_OK) r = q4::launch_gemv(fmt, L[i].qkv, st->h, st->qkv, qkv_n, hd, 1, s);
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
        if (r == Q4_OK) {
            hipLaunchKernelGGL(add_rmsnorm_kernel, dim3(1), dim3(kThreads), 0, s, st->x, st->delta, L[i].norm_mlp, st->h,
                               c->hidden, c->norm_eps);
            r = ok(hipGetLastError());
        }
        if (r == Q4_OK) r = q4::launch_gemv_glu(fmt, L[i].gate_up, st->h, st->act, c->ffn, hd, 1, s);
        if (r == Q4_OK) r = q4::launch_gemv(fmt, L[i].down, st->act, st->delta, hd, c->ffn, 1, s);
    }
    if (r != Q4_OK) return r;
    hipLaunchKernelGGL(add_rmsnorm_kernel, dim3(1), dim3(kThreads), 0, s, st->x, st->delta, norm_final, st->h, c->hidden,
                       c->norm_eps);
    r = ok(hipGetLastError());
    if (r == Q4_OK) r = q4::launch_gemv(fmt, emb, st->h, st->logits, c->vocab, hd, 1, s);
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
