// gdn_abi.cpp - the C ABI of libgdn.so: argument validation, error reporting and dispatch.
//
// Every check runs on the host before anything is enqueued, so an error leaves all buffers
// untouched.  Errors are reported as a status code plus a thread-local message (the single
// error sink of lucebox-hub internal.h, set_last_error).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <string>
#include <vector>

#include "../../include/gdn.h"
#include "gdn_internal.h"

#define GDN_API extern "C" __attribute__((visibility("default")))

namespace {

thread_local std::string g_last_error;

int vfail(int code, const char *fmt, va_list ap)
{
    char buf[512];
    vsnprintf(buf, sizeof buf, fmt, ap);
    g_last_error = buf;
    return code;
}

int fail(int code, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vfail(code, fmt, ap);
    va_end(ap);
    return code;
}

int ok()
{
    g_last_error.clear();
    return GDN_OK;
}

int hip_fail(hipError_t e, const char *what)
{
    return fail(GDN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr uint32_t kKnownFlags = GDN_F_QK_NORM_SILU | GDN_F_CHECK_INDICES | GDN_F_DEFER_COMMIT;
constexpr size_t kMaxLds = 160 * 1024;

size_t channels(const gdn_dims &d) { return 2 * (size_t)d.n_kh * d.d_k + (size_t)d.n_vh * d.d_v; }

int check_dims(const gdn_dims *d)
{
    if (!d) return fail(GDN_ERR_ARG, "dims is NULL");
    if (d->d_conv != 4) return fail(GDN_ERR_SHAPE, "d_conv must be 4 (got %d)", d->d_conv);
    if (d->d_k != d->d_v) return fail(GDN_ERR_SHAPE, "d_k (%d) must equal d_v (%d)", d->d_k, d->d_v);
    if (d->d_k != 64 && d->d_k != 128) return fail(GDN_ERR_SHAPE, "head dim must be 64 or 128 (got %d)", d->d_k);
    if (d->n_kh <= 0 || d->n_vh <= 0) return fail(GDN_ERR_SHAPE, "head counts must be positive");
    if (d->n_vh % d->n_kh) return fail(GDN_ERR_SHAPE, "n_vh (%d) must be a multiple of n_kh (%d)", d->n_vh, d->n_kh);
    const int ratio = d->n_vh / d->n_kh;
    if (ratio * gdn::verify_waves_per_head(d->d_k) * 64 > 1024)
        return fail(GDN_ERR_SHAPE, "n_vh / n_kh = %d value heads per key head exceeds one workgroup", ratio);
    if (d->n_pool <= 0) return fail(GDN_ERR_SHAPE, "n_pool must be positive");
    if ((d->act_dtype != GDN_F32 && d->act_dtype != GDN_BF16) || (d->out_dtype != GDN_F32 && d->out_dtype != GDN_BF16))
        return fail(GDN_ERR_DTYPE, "act_dtype / out_dtype must be GDN_F32 or GDN_BF16");
    if (d->flags & ~kKnownFlags) return fail(GDN_ERR_ARG, "unknown flag bits 0x%x", d->flags & ~kKnownFlags);
    if (!(d->eps >= 0.0f) || d->eps > 1.0f) return fail(GDN_ERR_ARG, "eps must be in [0, 1]");
    return GDN_OK;
}

bool same_shape(const gdn_dims &a, const gdn_dims &b)
{
    return a.n_kh == b.n_kh && a.n_vh == b.n_vh && a.d_k == b.d_k && a.d_v == b.d_v && a.d_conv == b.d_conv &&
           a.n_pool == b.n_pool;
}

int check_capture(const gdn_capture *c, int mode, int n_tok, const gdn_dims *d)
{
    if (c->mode != mode) return fail(GDN_ERR_ARG, "capture mode %d does not match the call (%d)", c->mode, mode);
    if (!c->ssm || !c->conv) return fail(GDN_ERR_ARG, "capture buffers are NULL");
    if (!aligned16(c->ssm) || !aligned16(c->conv)) return fail(GDN_ERR_ARG, "capture buffers must be 16-byte aligned");
    if (c->t_cap < n_tok) return fail(GDN_ERR_RANGE, "n_tok %d exceeds capture capacity t_cap %d", n_tok, c->t_cap);
    if (!same_shape(c->dims, *d)) return fail(GDN_ERR_SHAPE, "capture dims differ from the call's dims");
    return GDN_OK;
}

// Host copy + validation of device index arrays (GDN_F_CHECK_INDICES).
int fetch_i32(const int32_t *dev, size_t n, hipStream_t st, std::vector<int32_t> &out)
{
    // A capturing stream can record neither the copy nor the wait, and trying would end the
    // caller's capture: refuse before touching the stream.
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(st, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone)
        return fail(GDN_ERR_ARG, "GDN_F_CHECK_INDICES copies indices to the host, which a capturing stream cannot do");
    out.resize(n);
    hipError_t e = hipMemcpyAsync(out.data(), dev, n * sizeof(int32_t), hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) return hip_fail(e, "index check copy");
    return GDN_OK;
}

int check_slots(const int32_t *slot_ids, int n, int n_pool, hipStream_t st)
{
    std::vector<int32_t> h;
    if (int r = fetch_i32(slot_ids, n, st, h)) return r;
    std::vector<char> seen(n_pool, 0);
    for (int i = 0; i < n; ++i) {
        if (h[i] < 0 || h[i] >= n_pool) return fail(GDN_ERR_RANGE, "slot_ids[%d] = %d outside [0, %d)", i, h[i], n_pool);
        if (seen[h[i]]) return fail(GDN_ERR_RANGE, "slot %d appears twice", h[i]);
        seen[h[i]] = 1;
    }
    return GDN_OK;
}

int check_parents(const int32_t *parent, int n_batch, int n_tok, hipStream_t st)
{
    std::vector<int32_t> h;
    if (int r = fetch_i32(parent, (size_t)n_batch * n_tok, st, h)) return r;
    for (int b = 0; b < n_batch; ++b) {
        if (h[(size_t)b * n_tok] != -1) return fail(GDN_ERR_RANGE, "parent[%d][0] must be -1 (root)", b);
        for (int i = 1; i < n_tok; ++i) {
            const int p = h[(size_t)b * n_tok + i];
            if (p < -1 || p >= i) return fail(GDN_ERR_RANGE, "parent[%d][%d] = %d outside [-1, %d)", b, i, p, i);
        }
    }
    return GDN_OK;
}

gdn::VerifyArgs make_args(const gdn_dims &d, int n_tok, int n_batch)
{
    gdn::VerifyArgs a{};
    a.n_kh = d.n_kh;
    a.n_vh = d.n_vh;
    a.d = d.d_k;
    a.n_pool = d.n_pool;
    a.T = n_tok;
    a.C = (int32_t)channels(d);
    a.eps = d.eps;
    a.n_batch = n_batch;
    return a;
}

}  // namespace

namespace gdn {
int abi_check_dims(const gdn_dims *d) { return check_dims(d); }
}  // namespace gdn

namespace {
// Chain verify, from the slots' states (resume == NULL) or from the capture positions in resume.
int verify_chain(const char *fn, const gdn_dims *dims, float *state, float *conv_state, const void *qkv,
                 const void *z, const void *alpha, const void *beta, const float *A_log, const float *dt_bias,
                 const float *conv_w, const float *norm_w, const gdn_capture *capture, void *out, int32_t n_tok,
                 const int32_t *slot_ids, const int32_t *resume, int32_t n_batch, void *stream)
{
    if (int r = check_dims(dims)) return r;
    const gdn_dims &d = *dims;
    if (!state || !conv_state || !qkv || !z || !alpha || !beta || !A_log || !dt_bias || !conv_w || !norm_w || !out ||
        !slot_ids)
        return fail(GDN_ERR_ARG, "%s: a required pointer is NULL", fn);
    if (!aligned16(state) || !aligned16(conv_state) || !aligned16(conv_w) || !aligned16(z) || !aligned16(qkv))
        return fail(GDN_ERR_ARG, "%s: state, conv_state, conv_w, qkv and z must be 16-byte aligned", fn);
    if (n_tok < 1) return fail(GDN_ERR_RANGE, "%s: n_tok must be >= 1 (got %d)", fn, n_tok);
    if (n_batch < 1 || n_batch > d.n_pool)
        return fail(GDN_ERR_RANGE, "%s: n_batch %d outside [1, n_pool = %d]", fn, n_batch, d.n_pool);
    if (capture)
        if (int r = check_capture(capture, GDN_CHAIN, n_tok, dims)) return r;
    if (resume && !capture)
        return fail(GDN_ERR_ARG, "%s: resuming from capture positions needs the capture", fn);
    if ((d.flags & GDN_F_DEFER_COMMIT) && !capture)
        return fail(GDN_ERR_ARG, "%s: GDN_F_DEFER_COMMIT needs the capture, which then holds the state", fn);
    if (gdn::verify_chain_lds_bytes(d.d_k, d.n_vh / d.n_kh, d.act_dtype == GDN_BF16) > kMaxLds)
        return fail(GDN_ERR_SHAPE, "%s: LDS tile exceeds 160 KiB", fn);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (d.flags & GDN_F_CHECK_INDICES) {
        if (int r = check_slots(slot_ids, n_batch, d.n_pool, st)) return r;
        if (resume) {
            std::vector<int32_t> h;
            if (int r = fetch_i32(resume, n_batch, st, h)) return r;
            for (int i = 0; i < n_batch; ++i)
                if (h[i] >= capture->t_cap)
                    return fail(GDN_ERR_RANGE, "%s: resume_idx[%d] = %d outside [-1, t_cap = %d)", fn, i, h[i],
                                capture->t_cap);
        }
    }

    gdn::VerifyArgs a = make_args(d, n_tok, n_batch);
    a.t_cap = capture ? capture->t_cap : 0;
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
    a.cap_ssm = capture ? capture->ssm : nullptr;
    a.cap_conv = capture ? capture->conv : nullptr;
    a.out = out;
    a.slot_ids = slot_ids;
    a.resume = resume;
    a.defer = (d.flags & GDN_F_DEFER_COMMIT) ? 1 : 0;
    gdn::LaunchCfg c{d.act_dtype == GDN_BF16, d.out_dtype == GDN_BF16, (d.flags & GDN_F_QK_NORM_SILU) != 0};
    if (hipError_t e = gdn::launch_verify_chain(a, c, st))
        return fail(GDN_ERR_HIP, "%s launch: %s", fn, hipGetErrorString(e));
    return ok();
}
}  // namespace

GDN_API int gdn_verify(const gdn_dims *dims, float *state, float *conv_state, const void *qkv, const void *z,
                       const void *alpha, const void *beta, const float *A_log, const float *dt_bias,
                       const float *conv_w, const float *norm_w, const gdn_capture *capture, void *out,
                       int32_t n_tok, const int32_t *slot_ids, int32_t n_batch, void *stream)
{
    return verify_chain("gdn_verify", dims, state, conv_state, qkv, z, alpha, beta, A_log, dt_bias, conv_w, norm_w,
                        capture, out, n_tok, slot_ids, nullptr, n_batch, stream);
}

GDN_API int gdn_verify_resume(const gdn_dims *dims, float *state, float *conv_state, const void *qkv, const void *z,
                              const void *alpha, const void *beta, const float *A_log, const float *dt_bias,
                              const float *conv_w, const float *norm_w, const gdn_capture *capture, void *out,
                              int32_t n_tok, const int32_t *slot_ids, const int32_t *resume_idx, int32_t n_batch,
                              void *stream)
{
    if (!resume_idx) return fail(GDN_ERR_ARG, "gdn_verify_resume: resume_idx is NULL");
    if (!capture) return fail(GDN_ERR_ARG, "gdn_verify_resume: capture is NULL");
    return verify_chain("gdn_verify_resume", dims, state, conv_state, qkv, z, alpha, beta, A_log, dt_bias, conv_w,
                        norm_w, capture, out, n_tok, slot_ids, resume_idx, n_batch, stream);
}

GDN_API int gdn_verify_tree(const gdn_dims *dims, const float *state, const float *conv_state, const void *qkv,
                            const void *z, const void *alpha, const void *beta, const float *A_log,
                            const float *dt_bias, const float *conv_w, const float *norm_w, const int32_t *parent,
                            const gdn_capture *capture, void *out, int32_t n_tok, const int32_t *slot_ids,
                            int32_t n_batch, void *stream)
{
    if (int r = check_dims(dims)) return r;
    const gdn_dims &d = *dims;
    if (!state || !conv_state || !qkv || !z || !alpha || !beta || !A_log || !dt_bias || !conv_w || !norm_w ||
        !parent || !capture || !out || !slot_ids)
        return fail(GDN_ERR_ARG, "gdn_verify_tree: a required pointer is NULL");
    if (!aligned16(state) || !aligned16(conv_state) || !aligned16(conv_w) || !aligned16(qkv))
        return fail(GDN_ERR_ARG, "gdn_verify_tree: state, conv_state, conv_w and qkv must be 16-byte aligned");
    if (n_tok < 1) return fail(GDN_ERR_RANGE, "gdn_verify_tree: n_tok must be >= 1 (got %d)", n_tok);
    if (n_batch < 1 || n_batch > d.n_pool)
        return fail(GDN_ERR_RANGE, "gdn_verify_tree: n_batch %d outside [1, n_pool = %d]", n_batch, d.n_pool);
    if (int r = check_capture(capture, GDN_TREE, n_tok, dims)) return r;
    if (gdn::verify_tree_lds_bytes(d.d_k, n_tok, d.act_dtype == GDN_BF16) > kMaxLds)
        return fail(GDN_ERR_SHAPE, "gdn_verify_tree: %d nodes: at most 1024 per call", n_tok);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (d.flags & GDN_F_CHECK_INDICES) {
        if (int r = check_slots(slot_ids, n_batch, d.n_pool, st)) return r;
        if (int r = check_parents(parent, n_batch, n_tok, st)) return r;
    }
    gdn::VerifyArgs a = make_args(d, n_tok, n_batch);
    a.t_cap = capture->t_cap;
    a.state = const_cast<float *>(state);
    a.conv_state = const_cast<float *>(conv_state);
    a.qkv = qkv;
    a.z = z;
    a.alpha = alpha;
    a.beta = beta;
    a.A_log = A_log;
    a.dt_bias = dt_bias;
    a.conv_w = conv_w;
    a.norm_w = norm_w;
    a.cap_ssm = capture->ssm;
    a.cap_conv = capture->conv;
    a.out = out;
    a.slot_ids = slot_ids;
    a.parent = parent;
    gdn::LaunchCfg c{d.act_dtype == GDN_BF16, d.out_dtype == GDN_BF16, (d.flags & GDN_F_QK_NORM_SILU) != 0};
    if (hipError_t e = gdn::launch_verify_tree(a, c, st)) return hip_fail(e, "gdn_verify_tree launch");
    return ok();
}

namespace {

int check_rollback_capture(const gdn_capture *c)
{
    if (!c) return fail(GDN_ERR_ARG, "capture is NULL");
    if (int r = check_dims(&c->dims)) return r;
    if (!c->ssm || !c->conv || !c->state || !c->conv_state) return fail(GDN_ERR_ARG, "capture pointers are NULL");
    if (!aligned16(c->ssm) || !aligned16(c->conv) || !aligned16(c->state) || !aligned16(c->conv_state))
        return fail(GDN_ERR_ARG, "capture buffers must be 16-byte aligned");
    if (c->mode != GDN_CHAIN && c->mode != GDN_TREE) return fail(GDN_ERR_ARG, "capture mode must be CHAIN or TREE");
    if (c->t_cap < 1) return fail(GDN_ERR_RANGE, "capture t_cap must be >= 1");
    return GDN_OK;
}

gdn::RollbackArgs rollback_args(const gdn_capture *c)
{
    gdn::RollbackArgs a{};
    const gdn_dims &d = c->dims;
    a.state = c->state;
    a.conv_state = c->conv_state;
    a.cap_ssm = c->ssm;
    a.cap_conv = c->conv;
    a.n_pool = d.n_pool;
    a.t_cap = c->t_cap;
    a.mode = c->mode;
    a.C = channels(d);
    a.ssm_elems = (size_t)d.n_vh * d.d_v * d.d_k;
    a.conv_elems = 3 * a.C;
    return a;
}

}  // namespace

GDN_API int gdn_rollback(const gdn_capture *capture, int32_t slot, int32_t accepted_idx, void *stream)
{
    if (int r = check_rollback_capture(capture)) return r;
    if (slot < 0 || slot >= capture->dims.n_pool)
        return fail(GDN_ERR_RANGE, "gdn_rollback: slot %d outside [0, %d)", slot, capture->dims.n_pool);
    if (accepted_idx < 0 || accepted_idx >= capture->t_cap)
        return fail(GDN_ERR_RANGE, "gdn_rollback: accepted_idx %d outside [0, t_cap = %d)", accepted_idx, capture->t_cap);
    gdn::RollbackArgs a = rollback_args(capture);
    a.slot0 = slot;
    a.idx0 = accepted_idx;
    a.n = 1;
    if (hipError_t e = gdn::launch_rollback(a, static_cast<hipStream_t>(stream))) return hip_fail(e, "gdn_rollback launch");
    return ok();
}

GDN_API int gdn_rollback_batch(const gdn_capture *capture, const int32_t *slots, const int32_t *accepted_idx,
                               int32_t n, void *stream)
{
    if (int r = check_rollback_capture(capture)) return r;
    if (n < 0 || n > capture->dims.n_pool || n > 65535)
        return fail(GDN_ERR_RANGE, "gdn_rollback_batch: n = %d outside [0, min(n_pool = %d, 65535)]", n,
                    capture->dims.n_pool);
    if (n == 0) return ok();
    if (!slots || !accepted_idx) return fail(GDN_ERR_ARG, "gdn_rollback_batch: index arrays are NULL");
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (capture->dims.flags & GDN_F_CHECK_INDICES) {
        if (int r = check_slots(slots, n, capture->dims.n_pool, st)) return r;
        std::vector<int32_t> h;
        if (int r = fetch_i32(accepted_idx, n, st, h)) return r;
        for (int i = 0; i < n; ++i)
            if (h[i] < 0 || h[i] >= capture->t_cap)
                return fail(GDN_ERR_RANGE, "accepted_idx[%d] = %d outside [0, %d)", i, h[i], capture->t_cap);
    }
    gdn::RollbackArgs a = rollback_args(capture);
    a.slots = slots;
    a.idx = accepted_idx;
    a.n = n;
    if (hipError_t e = gdn::launch_rollback(a, st)) return hip_fail(e, "gdn_rollback_batch launch");
    return ok();
}

namespace {
bool same_geometry(const gdn_capture &a, const gdn_capture &b)
{
    const gdn_dims &x = a.dims, &y = b.dims;
    return x.n_kh == y.n_kh && x.n_vh == y.n_vh && x.d_k == y.d_k && x.d_v == y.d_v && x.d_conv == y.d_conv &&
           x.n_pool == y.n_pool && a.t_cap == b.t_cap && a.mode == b.mode;
}
}  // namespace

GDN_API int gdn_rollback_layers(const gdn_capture *layers, int32_t n_layers, const int32_t *slots,
                                const int32_t *accepted_idx, int32_t n, void *stream)
{
    if (!layers) return fail(GDN_ERR_ARG, "gdn_rollback_layers: layers is NULL");
    if (n_layers < 1) return fail(GDN_ERR_RANGE, "gdn_rollback_layers: n_layers = %d < 1", n_layers);
    const gdn_capture &l0 = layers[0];
    std::vector<const float *> owned;
    owned.reserve(2 * (size_t)n_layers);
    for (int l = 0; l < n_layers; ++l) {
        if (int r = check_rollback_capture(&layers[l])) return fail(r, "gdn_rollback_layers: layer %d: %s", l, gdn_last_error());
        if (!same_geometry(l0, layers[l]))
            return fail(GDN_ERR_ARG, "gdn_rollback_layers: layer %d differs from layer 0 in dims, t_cap or mode", l);
        owned.push_back(layers[l].state);
        owned.push_back(layers[l].conv_state);
    }
    std::sort(owned.begin(), owned.end());
    if (std::adjacent_find(owned.begin(), owned.end()) != owned.end())
        return fail(GDN_ERR_ARG, "gdn_rollback_layers: two layers share a state or conv_state buffer");
    if (n < 0 || n > l0.dims.n_pool || n > 65535)
        return fail(GDN_ERR_RANGE, "gdn_rollback_layers: n = %d outside [0, min(n_pool = %d, 65535)]", n, l0.dims.n_pool);
    if (n == 0) return ok();
    if (!slots || !accepted_idx) return fail(GDN_ERR_ARG, "gdn_rollback_layers: index arrays are NULL");
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (l0.dims.flags & GDN_F_CHECK_INDICES) {
        if (int r = check_slots(slots, n, l0.dims.n_pool, st)) return r;
        std::vector<int32_t> h;
        if (int r = fetch_i32(accepted_idx, n, st, h)) return r;
        for (int i = 0; i < n; ++i)
            if (h[i] < 0 || h[i] >= l0.t_cap)
                return fail(GDN_ERR_RANGE, "accepted_idx[%d] = %d outside [0, %d)", i, h[i], l0.t_cap);
    }
    gdn::RollbackLayersArgs a{};
    a.geo = rollback_args(&l0);
    a.geo.state = nullptr;
    a.geo.conv_state = nullptr;
    a.geo.cap_ssm = nullptr;
    a.geo.cap_conv = nullptr;
    a.geo.slots = slots;
    a.geo.idx = accepted_idx;
    a.geo.n = n;
    for (int l0i = 0; l0i < n_layers; l0i += gdn::kMaxLayersPerLaunch) {
        a.n_layers = n_layers - l0i < gdn::kMaxLayersPerLaunch ? n_layers - l0i : gdn::kMaxLayersPerLaunch;
        for (int j = 0; j < a.n_layers; ++j) {
            const gdn_capture &c = layers[l0i + j];
            a.layer[j] = gdn::LayerBuffers{c.state, c.conv_state, c.ssm, c.conv};
        }
        if (hipError_t e = gdn::launch_rollback_layers(a, st)) return hip_fail(e, "gdn_rollback_layers launch");
    }
    return ok();
}

GDN_API int gdn_rollback_trim(const gdn_capture *capture, int32_t slot, int32_t trim, int32_t n_tok, void *stream)
{
    if (int r = check_rollback_capture(capture)) return r;
    if (capture->mode != GDN_CHAIN)  // tree node indices are not positions along one path
        return fail(GDN_ERR_ARG, "gdn_rollback_trim: the trim form needs a GDN_CHAIN capture");
    if (n_tok < 1 || n_tok > capture->t_cap)
        return fail(GDN_ERR_RANGE, "gdn_rollback_trim: n_tok %d outside [1, t_cap = %d]", n_tok, capture->t_cap);
    if (trim < 0) return fail(GDN_ERR_RANGE, "gdn_rollback_trim: negative trim %d", trim);
    if (slot < 0 || slot >= capture->dims.n_pool)
        return fail(GDN_ERR_RANGE, "gdn_rollback_trim: slot %d outside [0, %d)", slot, capture->dims.n_pool);
    if (trim == 0) {
        // Nothing rejected.  A committing verify already left the final state; one that deferred
        // its commit left it at capture position n_tok - 1, which is restored here.
        if (!(capture->dims.flags & GDN_F_DEFER_COMMIT)) return ok();
        return gdn_rollback(capture, slot, n_tok - 1, stream);
    }
    if (trim >= n_tok)
        return fail(GDN_ERR_RANGE, "gdn_rollback_trim: trim %d >= verified positions %d", trim, n_tok);
    return gdn_rollback(capture, slot, n_tok - 1 - trim, stream);
}

GDN_API size_t gdn_capture_bytes(const gdn_dims *dims, int32_t t_cap, int32_t mode, size_t *conv_bytes)
{
    if (conv_bytes) *conv_bytes = 0;
    if (check_dims(dims) || t_cap < 1 || (mode != GDN_CHAIN && mode != GDN_TREE)) return 0;
    const gdn_dims &d = *dims;
    const size_t C = channels(d);
    if (conv_bytes)
        *conv_bytes = sizeof(float) * (size_t)d.n_pool * (mode == GDN_CHAIN ? (3 + (size_t)t_cap) * C : (size_t)t_cap * 3 * C);
    return sizeof(float) * (size_t)d.n_pool * t_cap * d.n_vh * d.d_v * d.d_k;
}

GDN_API int gdn_reset(const gdn_dims *dims, float *state, float *conv_state, int32_t slot, void *stream)
{
    if (int r = check_dims(dims)) return r;
    if (!state || !conv_state) return fail(GDN_ERR_ARG, "gdn_reset: NULL buffer");
    if (!aligned16(state) || !aligned16(conv_state)) return fail(GDN_ERR_ARG, "gdn_reset: buffers must be 16-byte aligned");
    if (slot < 0 || slot >= dims->n_pool) return fail(GDN_ERR_RANGE, "gdn_reset: slot %d outside [0, %d)", slot, dims->n_pool);
    const size_t ns = (size_t)dims->n_vh * dims->d_v * dims->d_k, nc = 3 * channels(*dims);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (hipError_t e = gdn::launch_fill_zero(state + (size_t)slot * ns, ns, st)) return hip_fail(e, "gdn_reset");
    if (hipError_t e = gdn::launch_fill_zero(conv_state + (size_t)slot * nc, nc, st)) return hip_fail(e, "gdn_reset");
    return ok();
}

namespace {
int slot_copy(const char *who, const gdn_dims *dims, float *dst_s, float *dst_c, const float *src_s, const float *src_c,
              const int32_t *slots, int32_t n, void *stream)
{
    if (int r = check_dims(dims)) return r;
    if (n < 0 || n > dims->n_pool || n > 65535)
        return fail(GDN_ERR_RANGE, "%s: n = %d outside [0, min(n_pool = %d, 65535)]", who, n, dims->n_pool);
    if (n == 0) return ok();
    if (!dst_s || !dst_c || !src_s || !src_c || !slots) return fail(GDN_ERR_ARG, "%s: NULL buffer or slot array", who);
    if (!aligned16(dst_s) || !aligned16(dst_c) || !aligned16(src_s) || !aligned16(src_c))
        return fail(GDN_ERR_ARG, "%s: state buffers must be 16-byte aligned", who);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (dims->flags & GDN_F_CHECK_INDICES)
        if (int r = check_slots(slots, n, dims->n_pool, st)) return r;
    gdn::SlotCopyArgs a{};
    a.dst_state = dst_s;
    a.dst_conv = dst_c;
    a.src_state = src_s;
    a.src_conv = src_c;
    a.slots = slots;
    a.n = n;
    a.n_pool = dims->n_pool;
    a.ssm_elems = (size_t)dims->n_vh * dims->d_v * dims->d_k;
    a.conv_elems = 3 * channels(*dims);
    if (hipError_t e = gdn::launch_slot_copy(a, st)) return hip_fail(e, who);
    return ok();
}
}  // namespace

GDN_API int gdn_snapshot(const gdn_dims *dims, const float *state, const float *conv_state, float *snap_state,
                         float *snap_conv, const int32_t *slots, int32_t n, void *stream)
{
    return slot_copy("gdn_snapshot", dims, snap_state, snap_conv, state, conv_state, slots, n, stream);
}

GDN_API int gdn_restore(const gdn_dims *dims, float *state, float *conv_state, const float *snap_state,
                        const float *snap_conv, const int32_t *slots, int32_t n, void *stream)
{
    return slot_copy("gdn_restore", dims, state, conv_state, snap_state, snap_conv, slots, n, stream);
}

namespace gdn {
int abi_fail(int code, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vfail(code, fmt, ap);
    va_end(ap);
    return code;
}
int abi_ok() { return ok(); }
}  // namespace gdn

GDN_API const char *gdn_last_error(void) { return g_last_error.c_str(); }

GDN_API const char *gdn_version(void) { return "gdn 0.1 (gfx950)"; }
