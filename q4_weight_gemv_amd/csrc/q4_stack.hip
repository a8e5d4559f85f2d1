// Layer-stack decode step: a list of decode products enqueued back-to-back on
// one stream, either launched directly or captured once into a HIP graph and
// replayed with a single launch per step.
//
// The runtime the pages describe batches kernel submissions, avoids CPU-GPU
// synchronisation, and caches compiled pipelines after the first forward pass
// (Llamas on the Web, technical summary, Methodology section 2, "execution
// scheduling"). On gfx950 the code objects are compiled ahead of time; the
// graph removes the per-launch host work of every step after the first.
#include <hip/hip_runtime.h>

#include <new>

#include "q4_internal.h"

struct q4_graph {
    hipGraph_t graph = nullptr;
    hipGraphExec_t exec = nullptr;
};

namespace {

int check_ops(int fmt, const q4_gemv_op *ops, int count, int64_t n)
{
    if (count < 0 || (count > 0 && !ops)) return Q4_EINVAL;
    for (int i = 0; i < count; i++) {
        int st = Q4_EINVAL;
        if (ops[i].epilogue == Q4_EPILOGUE_NONE)
            st = q4::check_product_args(fmt, ops[i].w, ops[i].x, ops[i].y, ops[i].m, ops[i].k, n, 8);
        else if (ops[i].epilogue == Q4_EPILOGUE_SILU_MUL)
            st = q4::check_glu_args(fmt, ops[i].w, ops[i].x, ops[i].y, ops[i].m, ops[i].k, n);
        if (st != Q4_OK) return st;
    }
    return Q4_OK;
}

int enqueue_ops(int fmt, const q4_gemv_op *ops, int count, int64_t n, hipStream_t s)
{
    for (int i = 0; i < count; i++) {
        if (ops[i].m == 0 || n == 0) continue;
        const int st = ops[i].epilogue == Q4_EPILOGUE_SILU_MUL
                           ? q4::launch_gemv_glu(fmt, ops[i].w, ops[i].x, ops[i].y, ops[i].m, ops[i].k, n, s)
                           : q4::launch_gemv(fmt, ops[i].w, ops[i].x, ops[i].y, ops[i].m, ops[i].k, n, s);
        if (st != Q4_OK) return st;
    }
    return Q4_OK;
}

}  // namespace

extern "C" {

int q4_gemv_sequence(int fmt, const q4_gemv_op *ops, int count, int64_t n, void *hip_stream)
{
    const int st = check_ops(fmt, ops, count, n);
    if (st != Q4_OK) return st;
    return enqueue_ops(fmt, ops, count, n, static_cast<hipStream_t>(hip_stream));
}

int q4_graph_create(int fmt, const q4_gemv_op *ops, int count, int64_t n, void *hip_stream, q4_graph **graph_out)
{
    if (!graph_out) return Q4_EINVAL;
    *graph_out = nullptr;
    int st = check_ops(fmt, ops, count, n);
    if (st != Q4_OK) return st;
    // Capture needs a non-null stream; use a private one if none is given.
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    hipStream_t own = nullptr;
    if (!s) {
        const int cst = q4::hip_status(hipStreamCreateWithFlags(&own, hipStreamNonBlocking));
        if (cst != Q4_OK) return cst;
        s = own;
    }
    q4_graph *g = new (std::nothrow) q4_graph();
    if (!g) {
        if (own) (void)hipStreamDestroy(own);
        return Q4_EHIP;
    }
    st = q4::hip_status(hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal));
    if (st == Q4_OK) {
        const int est = enqueue_ops(fmt, ops, count, n, s);
        const int end = q4::hip_status(hipStreamEndCapture(s, &g->graph));
        if (est != Q4_OK)
            st = est;
        else if (end != Q4_OK)
            st = end;
        else
            st = q4::hip_status(hipGraphInstantiate(&g->exec, g->graph, nullptr, nullptr, 0));
    }
    if (own) (void)hipStreamDestroy(own);
    if (st != Q4_OK) {
        q4_graph_destroy(g);
        return st;
    }
    *graph_out = g;
    return Q4_OK;
}

int q4_graph_launch(q4_graph *graph, void *hip_stream)
{
    if (!graph || !graph->exec) return Q4_EINVAL;
    return q4::hip_status(hipGraphLaunch(graph->exec, static_cast<hipStream_t>(hip_stream)));
}

int q4_graph_destroy(q4_graph *graph)
{
    if (!graph) return Q4_OK;
    int st = Q4_OK;
    if (graph->exec && q4::hip_status(hipGraphExecDestroy(graph->exec)) != Q4_OK) st = Q4_EHIP;
    if (graph->graph && q4::hip_status(hipGraphDestroy(graph->graph)) != Q4_OK) st = Q4_EHIP;
    delete graph;
    return st;
}

}  // extern "C"
