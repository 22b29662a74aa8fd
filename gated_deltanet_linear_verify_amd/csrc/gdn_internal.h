// gdn_internal.h - launch interface between the C ABI (gdn_abi.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

struct gdn_dims;  // include/gdn.h

namespace gdn {

constexpr int kTokenTile = 16;  // tokens per LDS tile in the verify kernels

struct VerifyArgs {
    int32_t n_kh, n_vh, d, n_pool, T, t_cap, C;
    int32_t t0, nt;  // chain verify: first token and token count of one launch (set by the launcher)
    float eps;
    float *state;
    float *conv_state;
    const void *qkv, *z, *alpha, *beta;
    const float *A_log, *dt_bias, *conv_w, *norm_w;
    float *cap_ssm;   // NULL: no capture
    float *cap_conv;
    void *out;
    const int32_t *slot_ids;
    const int32_t *resume;  // chain verify with capture: per batch entry, the capture position whose
                            // state and conv window the first token starts from (< 0: the slot's
                            // state); NULL: every entry starts from the slot's state
    const int32_t *parent;  // tree only
    int32_t n_batch;
    int32_t defer;  // chain verify with capture: leave state and conv_state untouched (the state
                    // after the last token stays at its capture position)
    int32_t hpw;    // chain verify: value heads per workgroup, set by the launcher (H_v/H_k, or 1)
    float *oscr;    // chain verify, row split: the launch's readout [n_batch][16][H_v][d] (set by the launcher)
};

// The row-split verify's readout scratch for stream st on the current device: the buffer kept for
// the stream (while st is capturing, only one reserved for capture), else (allocate, and st not
// capturing) a new one of kSplitScratchBytes, else NULL.
constexpr size_t kSplitScratchBytes = size_t(4) << 20;
void *split_scratch(hipStream_t st, bool allocate);
// Keep a buffer for st that launches under a capture on st may use (allocated now if st has none
// and is not capturing); false if there is none.
bool split_scratch_reserve(hipStream_t st);
// Remove the buffer kept for st and hand it to the caller (who frees it), or NULL.
void *split_scratch_take(hipStream_t st);

struct LaunchCfg {
    bool act_bf16, out_bf16, qk_norm;
};

// Chain verify: grid B * H_k workgroups of (H_v/H_k) * waves_per_head(d) waves.
hipError_t launch_verify_chain(const VerifyArgs &a, const LaunchCfg &c, hipStream_t stream);
// Tree verify: grid B * H_v workgroups of 2 * waves_per_head(d) waves; at most 64 nodes.
hipError_t launch_verify_tree(const VerifyArgs &a, const LaunchCfg &c, hipStream_t stream);

int verify_waves_per_head(int d);
size_t verify_chain_lds_bytes(int d, int ratio, bool act_bf16);
size_t verify_tree_lds_bytes(int d, int T, bool act_bf16);  // (size_t)-1 above the node limit

struct RollbackArgs {
    float *state, *conv_state;
    const float *cap_ssm, *cap_conv;
    int32_t n_pool, t_cap, mode;
    size_t ssm_elems;   // H_v * d_v * d_k floats per slot and position
    size_t conv_elems;  // 3 * C floats
    size_t C;
    const int32_t *slots;  // device array, or NULL: use slot0 / idx0
    const int32_t *idx;
    int32_t slot0, idx0, n;
};
hipError_t launch_rollback(const RollbackArgs &a, hipStream_t stream);

// Rollback of several layers' captures in one launch: the shapes, slots and indices are shared
// (geo; its buffer pointers are unused), each layer brings its own four buffers.
constexpr int kMaxLayersPerLaunch = 64;
struct LayerBuffers {
    float *state, *conv_state;
    const float *cap_ssm, *cap_conv;
};
struct RollbackLayersArgs {
    RollbackArgs geo;
    int32_t n_layers;  // 1 .. kMaxLayersPerLaunch
    LayerBuffers layer[kMaxLayersPerLaunch];
};
hipError_t launch_rollback_layers(const RollbackLayersArgs &a, hipStream_t stream);

hipError_t launch_fill_zero(float *p, size_t n, hipStream_t stream);

// Snapshot / restore: for each listed slot, copy its state and conv state from one pool-shaped
// pair of buffers to another.
struct SlotCopyArgs {
    float *dst_state, *dst_conv;
    const float *src_state, *src_conv;
    const int32_t *slots;  // device array of n slots; entries outside [0, n_pool) are skipped
    int32_t n, n_pool;
    size_t ssm_elems;   // H_v * d_v * d_k floats per slot
    size_t conv_elems;  // 3 * C floats per slot
};
hipError_t launch_slot_copy(const SlotCopyArgs &a, hipStream_t stream);

// Projections y = x W^T (bf16 in, fp32 accumulate): product columns [n0, n1) of segment s go to
// seg[s].ptr[m * ld + n - n0], as bf16 or fp32, optionally through a sigmoid.
constexpr int kMaxLinearSegs = 4;
struct LinearSeg {
    int32_t n0, ld, bf16, sigmoid;
    void *ptr;
};
struct LinearArgs {
    const uint16_t *x;  // [M][K] bf16
    const uint16_t *w;  // [N][K] bf16
    int32_t M, N, K;    // K a multiple of 64
    int32_t n_segs;     // 1 .. kMaxLinearSegs, ascending n0, seg[0].n0 == 0
    LinearSeg seg[kMaxLinearSegs];
};
hipError_t launch_linear(const LinearArgs &a, hipStream_t stream);

// The C ABI's thread-local last error (gdn_last_error): set it and return code, or clear it and
// return GDN_OK.
int abi_fail(int code, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
int abi_ok();
// Validation of gdn_dims as every entry point does it (sets the last error; GDN_OK if valid).
int abi_check_dims(const gdn_dims *d);

struct PrefillArgs {
    int32_t n_kh, n_vh, d, T, C, slot;
    float eps;
    float *state, *conv_state;
    const void *qkv, *z, *alpha, *beta;
    const float *A_log, *dt_bias, *conv_w, *norm_w;
    void *out;
    float *ws;  // workspace of prefill_workspace_bytes(): per-chunk operands and the fp32 readout
};
// Chunked prefill: a chunk-parallel prep kernel (conv, gates, T = (I + A)^-1 and P per chunk and
// value head), a sequential scan over H_v * (d / 16) workgroups, then the norm epilogue.
hipError_t launch_prefill(const PrefillArgs &a, const LaunchCfg &c, hipStream_t stream);
size_t prefill_workspace_bytes(int d, int n_kh, int n_vh, int T);
size_t prefill_lds_bytes(int d, bool act_bf16);  // the larger of the two kernels' LDS
// Every check of a prefill call except the workspace's (sets the last error); on GDN_OK, a holds
// the launch arguments with ws unset and c the kernel configuration.
int prefill_prepare(const char *fn, const gdn_dims *dims, float *state, float *conv_state, const void *qkv,
                    const void *z, const void *alpha, const void *beta, const float *A_log, const float *dt_bias,
                    const float *conv_w, const float *norm_w, void *out, int32_t n_tok, int32_t slot, PrefillArgs &a,
                    LaunchCfg &c);

}  // namespace gdn
