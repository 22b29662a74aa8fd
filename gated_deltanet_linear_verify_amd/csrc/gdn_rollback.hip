// gdn_rollback.hip - restore a slot's recurrent and conv state from the per-position capture.
//
// The state after accepted position a is capture element a (lucebox-hub internal.h, struct
// DeltaNetCapture: rollback reads offset (commit_n - 1)); the conv state is rows
// [a+1 .. a+3] of the chain capture window (same struct: slice [commit_n .. commit_n+kernel-2])
// or the per-node 3-row record of a tree capture.  hf2q qwen35_target.rs, rollback_la_to copies
// capture[accepted_idx] back into the live recurrent and conv buffers.  Both are bitwise copies:
// one flat float4 stream per entry, HBM bound.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

// One entry's copy: ns float4 of recurrent state and nc float4 of conv state, spread over the
// gridDim.x blocks that share the entry, four loads in flight per thread.  Everything is written
// with store_stream: plain stores leave their lines dirty in the caches, and the next verify, which
// streams its 2 GiB capture, then pays for their write-back (measured: 441 vs 464 us per verify
// with plain state stores; streaming the last ~14% of the state and the conv state as well took
// another ~2 us off it).
__device__ __forceinline__ void copy_entry(const f4 *src_s, f4 *dst_s, size_t ns, const f4 *src_c, f4 *dst_c, size_t nc)
{
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (; i + 3 * stride < ns; i += 4 * stride) {
        const f4 v0 = src_s[i], v1 = src_s[i + stride], v2 = src_s[i + 2 * stride], v3 = src_s[i + 3 * stride];
        store_stream(dst_s + i, v0);
        store_stream(dst_s + i + stride, v1);
        store_stream(dst_s + i + 2 * stride, v2);
        store_stream(dst_s + i + 3 * stride, v3);
    }
    for (; i < ns; i += stride) store_stream(dst_s + i, src_s[i]);
    for (size_t j = (size_t)blockIdx.x * blockDim.x + threadIdx.x; j < nc; j += stride) store_stream(dst_c + j, src_c[j]);
}

// Sources of entry (slot, idx) in one layer's capture: the state after position idx, and the conv
// state that follows it (chain window rows idx+1 .. idx+3, or the tree node's 3-row record).
__device__ __forceinline__ void rollback_entry(const RollbackArgs &a, const float *cap_ssm, const float *cap_conv,
                                               float *state, float *conv_state, int slot, int idx)
{
    const f4 *src_s = reinterpret_cast<const f4 *>(cap_ssm + ((size_t)slot * a.t_cap + idx) * a.ssm_elems);
    f4 *dst_s = reinterpret_cast<f4 *>(state + (size_t)slot * a.ssm_elems);
    const float *csrc = a.mode == 0 ? cap_conv + ((size_t)slot * (3 + a.t_cap) + idx + 1) * a.C
                                    : cap_conv + ((size_t)slot * a.t_cap + idx) * a.conv_elems;
    copy_entry(src_s, dst_s, a.ssm_elems / 4, reinterpret_cast<const f4 *>(csrc),
               reinterpret_cast<f4 *>(conv_state + (size_t)slot * a.conv_elems), a.conv_elems / 4);
}

__global__ __launch_bounds__(256) void rollback_kernel(RollbackArgs a)
{
    const int n = blockIdx.y;
    const int slot = a.slots ? a.slots[n] : a.slot0;
    const int idx = a.idx ? a.idx[n] : a.idx0;
    if (slot < 0 || slot >= a.n_pool || idx < 0 || idx >= a.t_cap) return;  // uniform per block
    rollback_entry(a, a.cap_ssm, a.cap_conv, a.state, a.conv_state, slot, idx);
}

// Every layer of a model at once (hf2q qwen35_target.rs, rollback_kv walks the captures of all
// linear-attention layers for the slot): blockIdx.z picks the layer, blockIdx.y the entry.  The
// per-layer buffers travel in the kernel arguments, so no device-side table is needed.
__global__ __launch_bounds__(256) void rollback_layers_kernel(RollbackLayersArgs a)
{
    const int n = blockIdx.y;
    const int slot = a.geo.slots[n];
    const int idx = a.geo.idx[n];
    if (slot < 0 || slot >= a.geo.n_pool || idx < 0 || idx >= a.geo.t_cap) return;  // uniform per block
    const LayerBuffers &L = a.layer[blockIdx.z];
    rollback_entry(a.geo, L.cap_ssm, L.cap_conv, L.state, L.conv_state, slot, idx);
}

// Blocks per entry: sized by the state alone, so that (for states of a multiple of 1024 float4)
// every thread copies exactly four float4 of it in one unrolled step; the conv state's float4 go to
// the first threads.
static unsigned copy_blocks(size_t ssm_elems)
{
    const size_t vec = ssm_elems / 4;
    size_t blocks = (vec + 256 * 4 - 1) / (256 * 4);
    if (blocks > 512) blocks = 512;
    if (blocks < 1) blocks = 1;
    return (unsigned)blocks;
}

hipError_t launch_rollback(const RollbackArgs &a, hipStream_t stream)
{
    if (a.n <= 0) return hipSuccess;
    hipLaunchKernelGGL(rollback_kernel, dim3(copy_blocks(a.ssm_elems), (unsigned)a.n), dim3(256), 0,
                       stream, a);
    return hipGetLastError();
}

hipError_t launch_rollback_layers(const RollbackLayersArgs &a, hipStream_t stream)
{
    if (a.geo.n <= 0 || a.n_layers <= 0) return hipSuccess;
    if (a.n_layers > kMaxLayersPerLaunch) return hipErrorInvalidValue;
    hipLaunchKernelGGL(rollback_layers_kernel,
                       dim3(copy_blocks(a.geo.ssm_elems), (unsigned)a.geo.n, (unsigned)a.n_layers),
                       dim3(256), 0, stream, a);
    return hipGetLastError();
}

// Snapshot and restore of whole slots (lucebox-hub internal.h: snapshot_ssm_state and
// restore_ssm_state copy the recurrent and conv state to and from TargetCache's ssm_state_snap /
// conv_state_snap).  Same flat float4 stream as the rollback, between two pool-shaped buffers.
__global__ __launch_bounds__(256) void slot_copy_kernel(SlotCopyArgs a)
{
    const int slot = a.slots[blockIdx.y];
    if (slot < 0 || slot >= a.n_pool) return;  // uniform per block
    copy_entry(reinterpret_cast<const f4 *>(a.src_state + (size_t)slot * a.ssm_elems),
               reinterpret_cast<f4 *>(a.dst_state + (size_t)slot * a.ssm_elems), a.ssm_elems / 4,
               reinterpret_cast<const f4 *>(a.src_conv + (size_t)slot * a.conv_elems),
               reinterpret_cast<f4 *>(a.dst_conv + (size_t)slot * a.conv_elems), a.conv_elems / 4);
}

hipError_t launch_slot_copy(const SlotCopyArgs &a, hipStream_t stream)
{
    if (a.n <= 0) return hipSuccess;
    hipLaunchKernelGGL(slot_copy_kernel, dim3(copy_blocks(a.ssm_elems), (unsigned)a.n), dim3(256), 0,
                       stream, a);
    return hipGetLastError();
}

__global__ __launch_bounds__(256) void fill_zero_kernel(f4 *p, size_t n4)
{
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) p[i] = f4{0.f, 0.f, 0.f, 0.f};
}

__global__ void fill_zero_tail_kernel(float *p, size_t n)
{
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0.f;
}

// Zero n floats at p (p 16-byte aligned).  A kernel rather than hipMemsetAsync so the call can
// sit inside a captured graph.
hipError_t launch_fill_zero(float *p, size_t n, hipStream_t stream)
{
    const size_t n4 = n / 4;
    if (n4) {
        size_t blocks = (n4 + 255) / 256;
        if (blocks > 2048) blocks = 2048;
        hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, reinterpret_cast<f4 *>(p), n4);
    }
    if (n % 4) hipLaunchKernelGGL(fill_zero_tail_kernel, dim3(1), dim3(64), 0, stream, p + n4 * 4, n % 4);
    return hipGetLastError();
}

}  // namespace gdn
