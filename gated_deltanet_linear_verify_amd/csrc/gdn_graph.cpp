// gdn_graph.cpp - a spec-decode step over many GDN layers recorded once as a HIP graph.
//
// The step is the library's own entry points (gdn_verify per layer, then gdn_rollback_layers)
// issued on a private stream under stream capture, so the graph holds exactly the kernels an
// eager step would launch, with the same arguments.  Replaying it costs one launch from the host
// instead of one per layer and phase (lucebox dflash_draft_kv.h replays the draft's recorded
// graph each step; lucebox-hub internal.h counts graph launches per step as the cost to cut).
#include <hip/hip_runtime.h>

#include <vector>

#include "../../include/gdn.h"
#include "gdn_internal.h"

#define GDN_API extern "C" __attribute__((visibility("default")))

struct gdn_graph {
    hipGraph_t graph = nullptr;
    hipGraphExec_t exec = nullptr;
    hipEvent_t done = nullptr;  // recorded after every replay, so destroy can wait for the last
    void *oscr = nullptr;       // the row-split verify's readout scratch the recorded kernels use
};

namespace {

void release(gdn_graph *g)
{
    if (!g) return;
    if (g->exec) (void)hipGraphExecDestroy(g->exec);
    if (g->graph) (void)hipGraphDestroy(g->graph);
    if (g->done) (void)hipEventDestroy(g->done);
    if (g->oscr) (void)hipFree(g->oscr);
    delete g;
}

// Issue the step's calls on `st` (under capture).  Returns a GDN_* code; the entry points set the
// last error themselves.
int issue_step(const gdn_dims *dims, const gdn_layer *layers, int n_layers, int n_tok, const int32_t *slot_ids,
               int n_batch, const int32_t *accepted_idx, uint32_t phases, const std::vector<gdn_capture> &caps,
               hipStream_t st)
{
    if (phases & GDN_GRAPH_VERIFY)
        for (int l = 0; l < n_layers; ++l) {
            const gdn_layer &L = layers[l];
            if (int r = gdn_verify(dims, L.state, L.conv_state, L.qkv, L.z, L.alpha, L.beta, L.A_log, L.dt_bias,
                                   L.conv_w, L.norm_w, &caps[l], L.out, n_tok, slot_ids, n_batch, st))
                return gdn::abi_fail(r, "gdn_graph_create: layer %d verify: %s", l, gdn_last_error());
        }
    if (phases & GDN_GRAPH_ROLLBACK)
        if (int r = gdn_rollback_layers(caps.data(), n_layers, slot_ids, accepted_idx, n_batch, st))
            return gdn::abi_fail(r, "gdn_graph_create: rollback: %s", gdn_last_error());
    return GDN_OK;
}

}  // namespace

GDN_API int gdn_graph_create(const gdn_dims *dims, const gdn_layer *layers, int32_t n_layers, int32_t t_cap,
                             int32_t n_tok, const int32_t *slot_ids, int32_t n_batch,
                             const int32_t *accepted_idx, uint32_t phases, gdn_graph **graph)
{
    if (!graph) return gdn::abi_fail(GDN_ERR_ARG, "gdn_graph_create: graph is NULL");
    *graph = nullptr;
    if (!dims || !layers) return gdn::abi_fail(GDN_ERR_ARG, "gdn_graph_create: dims or layers is NULL");
    if (dims->flags & GDN_F_CHECK_INDICES)
        return gdn::abi_fail(GDN_ERR_ARG, "gdn_graph_create: GDN_F_CHECK_INDICES copies indices to the host and "
                                          "cannot be recorded");
    if (!phases || (phases & ~(GDN_GRAPH_VERIFY | GDN_GRAPH_ROLLBACK)))
        return gdn::abi_fail(GDN_ERR_ARG, "gdn_graph_create: phases 0x%x must be a non-empty set of GDN_GRAPH_* bits",
                             phases);
    if (n_layers < 1) return gdn::abi_fail(GDN_ERR_RANGE, "gdn_graph_create: n_layers = %d < 1", n_layers);
    if (t_cap < n_tok || n_tok < 1)
        return gdn::abi_fail(GDN_ERR_RANGE, "gdn_graph_create: need 1 <= n_tok (%d) <= t_cap (%d)", n_tok, t_cap);
    if ((phases & GDN_GRAPH_ROLLBACK) && !accepted_idx)
        return gdn::abi_fail(GDN_ERR_ARG, "gdn_graph_create: the rollback phase needs accepted_idx");
    for (int l = 0; l < n_layers; ++l) {
        const gdn_layer &L = layers[l];
        if (!L.state || !L.conv_state || !L.qkv || !L.z || !L.alpha || !L.beta || !L.A_log || !L.dt_bias || !L.conv_w ||
            !L.norm_w || !L.cap_ssm || !L.cap_conv || !L.out)
            return gdn::abi_fail(GDN_ERR_ARG, "gdn_graph_create: layer %d has a NULL buffer", l);
    }
    if (!slot_ids) return gdn::abi_fail(GDN_ERR_ARG, "gdn_graph_create: slot_ids is NULL");
    std::vector<gdn_capture> caps((size_t)n_layers);
    for (int l = 0; l < n_layers; ++l)
        caps[l] = gdn_capture{*dims, layers[l].cap_ssm, layers[l].cap_conv, layers[l].state, layers[l].conv_state,
                              t_cap, GDN_CHAIN};

    hipStream_t st = nullptr;
    if (hipError_t e = hipStreamCreateWithFlags(&st, hipStreamNonBlocking))
        return gdn::abi_fail(GDN_ERR_HIP, "gdn_graph_create: stream: %s", hipGetErrorString(e));
    gdn_graph *g = new gdn_graph;
    int rc = GDN_OK;
    // A readout scratch for the capture stream, kept by the graph: row-split verify launches under
    // the capture use it (without one they take the unsplit path).
    (void)gdn::split_scratch_reserve(st);
    if (hipError_t e = hipStreamBeginCapture(st, hipStreamCaptureModeThreadLocal)) {
        rc = gdn::abi_fail(GDN_ERR_HIP, "gdn_graph_create: begin capture: %s", hipGetErrorString(e));
    } else {
        rc = issue_step(dims, layers, n_layers, n_tok, slot_ids, n_batch, accepted_idx, phases, caps, st);
        const hipError_t ee = hipStreamEndCapture(st, &g->graph);  // always end, also after an error
        if (rc == GDN_OK && ee != hipSuccess)
            rc = gdn::abi_fail(GDN_ERR_HIP, "gdn_graph_create: end capture: %s", hipGetErrorString(ee));
    }
    g->oscr = gdn::split_scratch_take(st);
    if (rc == GDN_OK)
        if (hipError_t e = hipGraphInstantiate(&g->exec, g->graph, nullptr, nullptr, 0))
            rc = gdn::abi_fail(GDN_ERR_HIP, "gdn_graph_create: instantiate: %s", hipGetErrorString(e));
    if (rc == GDN_OK)
        if (hipError_t e = hipEventCreateWithFlags(&g->done, hipEventDisableTiming))
            rc = gdn::abi_fail(GDN_ERR_HIP, "gdn_graph_create: event: %s", hipGetErrorString(e));
    (void)hipStreamDestroy(st);
    if (rc != GDN_OK) {
        release(g);
        return rc;
    }
    *graph = g;
    return gdn::abi_ok();
}

GDN_API int gdn_graph_launch(const gdn_graph *graph, void *stream)
{
    if (!graph || !graph->exec) return gdn::abi_fail(GDN_ERR_ARG, "gdn_graph_launch: graph is NULL");
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (hipError_t e = hipGraphLaunch(graph->exec, st))
        return gdn::abi_fail(GDN_ERR_HIP, "gdn_graph_launch: %s", hipGetErrorString(e));
    if (hipError_t e = hipEventRecord(graph->done, st))
        return gdn::abi_fail(GDN_ERR_HIP, "gdn_graph_launch: event: %s", hipGetErrorString(e));
    return gdn::abi_ok();
}

GDN_API int gdn_graph_destroy(gdn_graph *graph)
{
    if (!graph) return gdn::abi_ok();
    hipError_t e = graph->done ? hipEventSynchronize(graph->done) : hipSuccess;
    release(graph);
    if (e != hipSuccess) return gdn::abi_fail(GDN_ERR_HIP, "gdn_graph_destroy: %s", hipGetErrorString(e));
    return gdn::abi_ok();
}
