// Captured decode step: the one-token decode of many layers (conv1d_update + state_update
// per layer) recorded once as a HIP graph and replayed with a single launch. A mixed
// prefill + decode iteration can then run its prefill segment eagerly and its decode rows
// as one replay (the split asked about on the TRT-LLM page, "Questions" item 1).
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <new>
#include <string>

#include "../../include/mamba2.h"

struct mamba2_decode_graph {
    hipGraph_t graph = nullptr;
    hipGraphExec_t exec = nullptr;
    int32_t nlayers = 0;
};

namespace {

// The entry points keep their message in a thread-local string of api.cpp; errors of the
// HIP graph calls themselves are reported through the same status codes with this text.
thread_local std::string g_graph_error;

int graph_fail(int status, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_graph_error = buf;
    return status;
}

}  // namespace

extern "C" {

int mamba2_decode_graph_create(const mamba2_dims *dims, const mamba2_decode_layer *layers, int32_t nlayers,
                               int32_t batch, void *capture_stream, mamba2_decode_graph **out) {
    g_graph_error.clear();
    if (!out) return graph_fail(MAMBA2_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    if (!dims || (!layers && nlayers > 0) || nlayers < 0 || batch < 0)
        return graph_fail(MAMBA2_ERR_INVALID_ARG, "dims/layers missing or negative nlayers/batch");
    if (!capture_stream)
        return graph_fail(MAMBA2_ERR_INVALID_ARG, "capture_stream must be a created stream, not the default stream");
    int st = mamba2_check_dims(dims);
    if (st) return st;
    hipStream_t s = static_cast<hipStream_t>(capture_stream);
    auto *g = new (std::nothrow) mamba2_decode_graph;
    if (!g) return graph_fail(MAMBA2_ERR_HIP, "out of host memory");
    g->nlayers = nlayers;
    hipError_t e = hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal);
    if (e != hipSuccess) {
        delete g;
        return graph_fail(MAMBA2_ERR_HIP, "hipStreamBeginCapture: %s", hipGetErrorString(e));
    }
    for (int32_t l = 0; l < nlayers && st == MAMBA2_OK; ++l) {
        const mamba2_decode_layer &L = layers[l];
        st = mamba2_conv1d_update(dims, L.xbc, L.conv_w, L.conv_b, L.xbc_post, L.conv_pool, L.num_slots,
                                  L.state_indices, batch, s);
        if (st == MAMBA2_OK)
            st = mamba2_state_update(dims, L.xbc_post, L.dt_raw, L.A_log, L.dt_bias, L.D, L.z, L.y, L.ssm_pool,
                                     L.num_slots, L.state_indices, batch, s);
        if (st) g_graph_error = std::string("layer ") + std::to_string(l) + ": " + mamba2_last_error();
    }
    hipGraph_t graph = nullptr;
    e = hipStreamEndCapture(s, &graph);  // always ends the capture, also after a failed layer
    if (st || e != hipSuccess) {
        if (graph) (void)hipGraphDestroy(graph);
        delete g;
        if (st) return st;
        return graph_fail(MAMBA2_ERR_HIP, "hipStreamEndCapture: %s", hipGetErrorString(e));
    }
    g->graph = graph;
    e = hipGraphInstantiateWithFlags(&g->exec, graph, 0);
    if (e != hipSuccess) {
        (void)hipGraphDestroy(graph);
        delete g;
        return graph_fail(MAMBA2_ERR_HIP, "hipGraphInstantiate: %s", hipGetErrorString(e));
    }
    *out = g;
    return MAMBA2_OK;
}

int mamba2_decode_graph_launch(mamba2_decode_graph *g, void *stream) {
    g_graph_error.clear();
    if (!g || !g->exec) return graph_fail(MAMBA2_ERR_INVALID_ARG, "graph is NULL");
    const hipError_t e = hipGraphLaunch(g->exec, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return graph_fail(MAMBA2_ERR_HIP, "hipGraphLaunch: %s", hipGetErrorString(e));
    return MAMBA2_OK;
}

void mamba2_decode_graph_destroy(mamba2_decode_graph *g) {
    if (!g) return;
    if (g->exec) (void)hipGraphExecDestroy(g->exec);
    if (g->graph) (void)hipGraphDestroy(g->graph);
    delete g;
}

const char *mamba2_decode_graph_last_error(void) { return g_graph_error.c_str(); }

}  // extern "C"
