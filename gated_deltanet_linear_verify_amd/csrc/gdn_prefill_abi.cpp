// gdn_prefill_abi.cpp - C ABI of the chunked prefill: validation and dispatch.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>

#include "../../include/gdn.h"
#include "gdn_internal.h"

#define GDN_API extern "C" __attribute__((visibility("default")))

namespace {
bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
constexpr size_t kMaxLds = 160 * 1024;
}  // namespace

GDN_API size_t gdn_prefill_workspace_bytes(const gdn_dims *dims, int32_t n_tok)
{
    if (gdn::abi_check_dims(dims) || n_tok < 1) return 0;
    return gdn::prefill_workspace_bytes(dims->d_v, dims->n_kh, dims->n_vh, n_tok);
}

namespace gdn {
// Every check of a prefill call except the workspace's, and the launch arguments (ws unset).
int prefill_prepare(const char *fn, const gdn_dims *dims, float *state, float *conv_state, const void *qkv,
                    const void *z, const void *alpha, const void *beta, const float *A_log, const float *dt_bias,
                    const float *conv_w, const float *norm_w, void *out, int32_t n_tok, int32_t slot, PrefillArgs &a,
                    LaunchCfg &c)
{
    if (int r = abi_check_dims(dims)) return r;
    const gdn_dims &d = *dims;
    if (!state || !conv_state || !qkv || !z || !alpha || !beta || !A_log || !dt_bias || !conv_w || !norm_w || !out)
        return abi_fail(GDN_ERR_ARG, "%s: a required pointer is NULL", fn);
    if (!aligned16(state) || !aligned16(conv_state) || !aligned16(conv_w) || !aligned16(qkv) || !aligned16(z) ||
        !aligned16(out) || !aligned16(norm_w))
        return abi_fail(GDN_ERR_ARG, "%s: state, conv_state, conv_w, qkv, z, out and norm_w must be 16-byte aligned",
                        fn);
    if (n_tok < 1) return abi_fail(GDN_ERR_RANGE, "%s: n_tok must be >= 1", fn);
    if (slot < 0 || slot >= d.n_pool) return abi_fail(GDN_ERR_RANGE, "%s: slot outside [0, n_pool)", fn);
    if (prefill_lds_bytes(d.d_k, d.act_dtype == GDN_BF16) > kMaxLds)
        return abi_fail(GDN_ERR_SHAPE, "%s: the kernels' LDS exceeds one workgroup's 160 KiB", fn);
    a = PrefillArgs{};
    a.n_kh = d.n_kh;
    a.n_vh = d.n_vh;
    a.d = d.d_k;
    a.T = n_tok;
    a.C = 2 * d.n_kh * d.d_k + d.n_vh * d.d_v;
    a.slot = slot;
    a.eps = d.eps;
    a.state = state;
    a.conv_state = conv_state;
    a.qkv = qkv;
    a.z = z;
    a.alpha = alpha;
    a.beta = beta;
    a.A_log = A_log;
    a.dt_bias = dt_bias;
    a.conv_w = conv_w;
    a.norm_w = norm_w;
    a.out = out;
    c = LaunchCfg{d.act_dtype == GDN_BF16, d.out_dtype == GDN_BF16, (d.flags & GDN_F_QK_NORM_SILU) != 0};
    return GDN_OK;
}
}  // namespace gdn

GDN_API int gdn_prefill(const gdn_dims *dims, float *state, float *conv_state, const void *qkv, const void *z,
                        const void *alpha, const void *beta, const float *A_log, const float *dt_bias,
                        const float *conv_w, const float *norm_w, void *out, int32_t n_tok, int32_t slot,
                        void *workspace, size_t ws_bytes, void *stream)
{
    gdn::PrefillArgs a;
    gdn::LaunchCfg c;
    if (int r = gdn::prefill_prepare("gdn_prefill", dims, state, conv_state, qkv, z, alpha, beta, A_log, dt_bias,
                                     conv_w, norm_w, out, n_tok, slot, a, c))
        return r;
    if (!workspace) return gdn::abi_fail(GDN_ERR_ARG, "gdn_prefill: workspace is NULL");
    if (!aligned16(workspace)) return gdn::abi_fail(GDN_ERR_ARG, "gdn_prefill: workspace must be 16-byte aligned");
    if (ws_bytes < gdn::prefill_workspace_bytes(dims->d_v, dims->n_kh, dims->n_vh, n_tok))
        return gdn::abi_fail(GDN_ERR_ARG, "gdn_prefill: workspace smaller than gdn_prefill_workspace_bytes()");
    a.ws = static_cast<float *>(workspace);
    if (hipError_t e = gdn::launch_prefill(a, c, static_cast<hipStream_t>(stream)))
        return gdn::abi_fail(GDN_ERR_HIP, "gdn_prefill launch: %s", hipGetErrorString(e));
    return gdn::abi_ok();
}
