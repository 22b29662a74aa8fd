// gdn_linear_abi.cpp - C ABI of the block's projections: validation and dispatch.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/gdn.h"
#include "gdn_internal.h"

#define GDN_API extern "C" __attribute__((visibility("default")))

GDN_API int gdn_linear(const void *x, const void *w, int32_t M, int32_t N, int32_t K, const gdn_out_seg *segs,
                       int32_t n_segs, void *stream)
{
    if (!x || !w || !segs) return gdn::abi_fail(GDN_ERR_ARG, "gdn_linear: x, w and segs must not be NULL");
    if (((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(w)) & 15u) != 0)
        return gdn::abi_fail(GDN_ERR_ARG, "gdn_linear: x and w must be 16-byte aligned");
    if (M < 1 || N < 1) return gdn::abi_fail(GDN_ERR_SHAPE, "gdn_linear: M = %d and N = %d must be >= 1", M, N);
    if (K < 64 || K % 64) return gdn::abi_fail(GDN_ERR_SHAPE, "gdn_linear: K = %d must be a positive multiple of 64", K);
    if (n_segs < 1 || n_segs > gdn::kMaxLinearSegs)
        return gdn::abi_fail(GDN_ERR_ARG, "gdn_linear: n_segs = %d outside [1, %d]", n_segs, gdn::kMaxLinearSegs);
    gdn::LinearArgs a{};
    a.x = static_cast<const uint16_t *>(x);
    a.w = static_cast<const uint16_t *>(w);
    a.M = M;
    a.N = N;
    a.K = K;
    a.n_segs = n_segs;
    int expect = 0;
    for (int s = 0; s < n_segs; ++s) {
        const gdn_out_seg &g = segs[s];
        if (g.n0 != expect || g.n1 <= g.n0)
            return gdn::abi_fail(GDN_ERR_ARG, "gdn_linear: segment %d covers [%d, %d), expected to start at %d", s,
                                 g.n0, g.n1, expect);
        if (!g.ptr) return gdn::abi_fail(GDN_ERR_ARG, "gdn_linear: segment %d has a NULL destination", s);
        if (g.ld < g.n1 - g.n0) return gdn::abi_fail(GDN_ERR_ARG, "gdn_linear: segment %d: ld %d < width %d", s, g.ld, g.n1 - g.n0);
        if (g.dtype != GDN_BF16 && g.dtype != GDN_F32)
            return gdn::abi_fail(GDN_ERR_DTYPE, "gdn_linear: segment %d: dtype must be GDN_BF16 or GDN_F32", s);
        a.seg[s] = gdn::LinearSeg{g.n0, g.ld, g.dtype == GDN_BF16, g.sigmoid != 0, g.ptr};
        expect = g.n1;
    }
    if (expect != N) return gdn::abi_fail(GDN_ERR_ARG, "gdn_linear: segments end at %d, not N = %d", expect, N);
    if (hipError_t e = gdn::launch_linear(a, static_cast<hipStream_t>(stream)))
        return gdn::abi_fail(GDN_ERR_HIP, "gdn_linear launch: %s", hipGetErrorString(e));
    return gdn::abi_ok();
}
