// gdn_noalloc.hip - gdn_prefill_noalloc: the chunked prefill with its workspace in a static device
// array, for callers that cannot allocate device memory (code under HIP graph capture, tight
// serving loops, harnesses that forbid hipMalloc).
//
// The array lives in this file's code object; each GPU the library runs on holds its own copy
// until the process ends.  Host code never passes the array's name to a kernel (on the host that
// name is only a stand-in, not a device address): the device address is looked up once per
// device with hipGetSymbolAddress, with that device current, and only that address is used.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/gdn.h"
#include "gdn_internal.h"

#define GDN_API extern "C" __attribute__((visibility("default")))

namespace {

constexpr size_t kScratchBytes = size_t(64) << 20;  // GDN_NOALLOC_SCRATCH_BYTES in gdn.h
static_assert(kScratchBytes == GDN_NOALLOC_SCRATCH_BYTES, "the header states the scratch size");

static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_ptr[kMaxDevices];  // device address of `scratch` on each device, once looked up

// The scratch's device address on the current device (looked up on the first call there).
int scratch_on_current_device(void **out)
{
    int dev = -1;
    if (hipError_t e = hipGetDevice(&dev))
        return gdn::abi_fail(GDN_ERR_HIP, "gdn_prefill_noalloc: hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return gdn::abi_fail(GDN_ERR_HIP, "gdn_prefill_noalloc: device %d beyond the %d this library tracks", dev,
                             kMaxDevices);
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[dev]) {
        void *p = nullptr;
        if (hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)))
            return gdn::abi_fail(GDN_ERR_HIP, "gdn_prefill_noalloc: hipGetSymbolAddress(scratch): %s",
                                 hipGetErrorString(e));
        if (!p || (reinterpret_cast<uintptr_t>(p) & 255u))
            return gdn::abi_fail(GDN_ERR_HIP, "gdn_prefill_noalloc: scratch address %p is not 256-byte aligned", p);
        g_ptr[dev] = p;
    }
    *out = g_ptr[dev];
    return GDN_OK;
}

size_t act_bytes(int dtype) { return dtype == GDN_BF16 ? 2 : 4; }

}  // namespace

GDN_API int gdn_prefill_noalloc(const gdn_dims *dims, float *state, float *conv_state, const void *qkv, const void *z,
                                const void *alpha, const void *beta, const float *A_log, const float *dt_bias,
                                const float *conv_w, const float *norm_w, void *out, int32_t n_tok, int32_t slot,
                                void *stream)
{
    gdn::PrefillArgs a;
    gdn::LaunchCfg c;
    if (int r = gdn::prefill_prepare("gdn_prefill_noalloc", dims, state, conv_state, qkv, z, alpha, beta, A_log,
                                     dt_bias, conv_w, norm_w, out, n_tok, slot, a, c))
        return r;
    const gdn_dims &d = *dims;
    // The workspace grows with whole 64-token chunks; a call runs as consecutive pieces of the most
    // chunks whose workspace fits the scratch (the state and conv state carry over between pieces
    // exactly as between two gdn_prefill calls).
    size_t piece = kScratchBytes / gdn::prefill_workspace_bytes(d.d_v, d.n_kh, d.n_vh, 64) * 64;
    while (piece > 0 && gdn::prefill_workspace_bytes(d.d_v, d.n_kh, d.n_vh, (int)piece) > kScratchBytes) piece -= 64;
    if (piece == 0)
        return gdn::abi_fail(GDN_ERR_SHAPE,
                             "gdn_prefill_noalloc: one 64-token chunk needs %zu workspace bytes, more than the %zu-byte "
                             "static scratch",
                             gdn::prefill_workspace_bytes(d.d_v, d.n_kh, d.n_vh, 64), kScratchBytes);
    void *ws = nullptr;
    if (int r = scratch_on_current_device(&ws)) return r;
    const size_t ab = act_bytes(d.act_dtype), ob = act_bytes(d.out_dtype);
    const size_t row_qkv = (size_t)a.C * ab, row_z = (size_t)d.n_vh * d.d_v * ab, row_g = (size_t)d.n_vh * ab,
                 row_out = (size_t)d.n_vh * d.d_v * ob;
    hipStream_t st = static_cast<hipStream_t>(stream);
    for (size_t t0 = 0; t0 < (size_t)n_tok; t0 += piece) {
        gdn::PrefillArgs p = a;
        p.T = (int32_t)((size_t)n_tok - t0 < piece ? (size_t)n_tok - t0 : piece);
        p.qkv = static_cast<const char *>(qkv) + t0 * row_qkv;
        p.z = static_cast<const char *>(z) + t0 * row_z;
        p.alpha = static_cast<const char *>(alpha) + t0 * row_g;
        p.beta = static_cast<const char *>(beta) + t0 * row_g;
        p.out = static_cast<char *>(out) + t0 * row_out;
        p.ws = static_cast<float *>(ws);
        if (hipError_t e = gdn::launch_prefill(p, c, st))
            return gdn::abi_fail(GDN_ERR_HIP, "gdn_prefill_noalloc launch: %s", hipGetErrorString(e));
    }
    return gdn::abi_ok();
}
