// gdn_prefill.cpp - chunked prefill entry points (placeholder until the kernels land).
#include <hip/hip_runtime.h>

#include "../../include/gdn.h"

#define GDN_API extern "C" __attribute__((visibility("default")))

GDN_API size_t gdn_prefill_workspace_bytes(const gdn_dims *, int32_t) { return 0; }

GDN_API int gdn_prefill(const gdn_dims *, float *, float *, const void *, const void *, const void *,
                        const void *, const float *, const float *, const float *, const float *, void *,
                        int32_t, int32_t, void *, size_t, void *)
{
    return GDN_ERR_SHAPE;
}
