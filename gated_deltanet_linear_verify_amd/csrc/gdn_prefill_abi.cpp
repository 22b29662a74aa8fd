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

GDN_API int gdn_prefill(const gdn_dims *dims, float *state, float *conv_state, const void *qkv, const void *z,
                        const void *alpha, const void *beta, const float *A_log, const float *dt_bias,
                        const float *conv_w, const float *norm_w, void *out, int32_t n_tok, int32_t slot,
                        void *workspace, size_t ws_bytes, void *stream)
{
    if (int r = gdn::abi_check_dims(dims)) return r;
    const gdn_dims &d = *dims;
    if (!state || !conv_state || !qkv || !z || !alpha || !beta || !A_log || !dt_bias || !conv_w || !norm_w || !out ||
        !workspace)
        return gdn::abi_fail(GDN_ERR_ARG, "gdn_prefill: a required pointer is NULL");
    if (!aligned16(state) || !aligned16(conv_state) || !aligned16(conv_w) || !aligned16(qkv) || !aligned16(workspace) ||
        !aligned16(z) || !aligned16(out) || !aligned16(norm_w))
        return gdn::abi_fail(GDN_ERR_ARG,
                             "gdn_prefill: state, conv_state, conv_w, qkv, z, out, norm_w and workspace must be 16-byte aligned");
    if (n_tok < 1) return gdn::abi_fail(GDN_ERR_RANGE, "gdn_prefill: n_tok must be >= 1");
    if (slot < 0 || slot >= d.n_pool) return gdn::abi_fail(GDN_ERR_RANGE, "gdn_prefill: slot outside [0, n_pool)");
    if (ws_bytes < gdn::prefill_workspace_bytes(d.d_v, d.n_kh, d.n_vh, n_tok))
        return gdn::abi_fail(GDN_ERR_ARG, "gdn_prefill: workspace smaller than gdn_prefill_workspace_bytes()");
    if (gdn::prefill_lds_bytes(d.d_k, d.act_dtype == GDN_BF16) > kMaxLds)
        return gdn::abi_fail(GDN_ERR_SHAPE, "gdn_prefill: the kernels' LDS exceeds one workgroup's 160 KiB");
    gdn::PrefillArgs a{};
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
    a.ws = static_cast<float *>(workspace);
    gdn::LaunchCfg c{d.act_dtype == GDN_BF16, d.out_dtype == GDN_BF16, (d.flags & GDN_F_QK_NORM_SILU) != 0};
    if (hipError_t e = gdn::launch_prefill(a, c, static_cast<hipStream_t>(stream)))
        return gdn::abi_fail(GDN_ERR_HIP, "gdn_prefill launch: %s", hipGetErrorString(e));
    return gdn::abi_ok();
}
