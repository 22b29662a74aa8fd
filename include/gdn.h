/*
 * gdn.h - C ABI of libgdn.so: the Gated DeltaNet speculative-decode verify path on AMD MI355X
 * (gfx950), as hand-written HIP kernels.
 *
 * What is computed (per slot s and value head h; the recurrent layer of a Qwen3.5-style hybrid
 * model, "GATED DELTANET block" in lucebox-hub server/src/internal.h, struct TargetLayer):
 *
 *   xext      = concat(conv_state[s] (3 rows, oldest first), qkv rows of the new tokens)
 *   xhat[t]   = sum_j conv_w[c][j] * xext[t + j]          depthwise causal conv, kernel 4, no bias
 *   q, k, v   = the q / k channels of key head h / (H_v / H_k) and the v channels of head h
 *   g_t       = -exp(A_log[h]) * softplus(alpha_t + dt_bias[h]),   rho_t = exp(g_t)
 *   S_t       = rho_t * S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *   o_t       = S_t q_t
 *   out_t     = o_t / sqrt(mean(o_t^2) + eps) * norm_w * z_t * sigmoid(z_t)
 *
 * (gated delta rule: Yang, Kautz & Hatamizadeh, "Gated Delta Networks", 2024; the parameter
 * tensors ssm_conv1d, ssm_a, ssm_dt_bias, ssm_beta, ssm_alpha, ssm_norm and the z projection
 * are listed in lucebox-hub internal.h, struct TargetLayer; rms_eps in struct TargetWeights.)
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Layouts are row-major, last index fastest.  C = 2*H_k*d_k + H_v*d_v conv channels, in
 *   blocks q [H_k][d_k] | k [H_k][d_k] | v [H_v][d_v].
 *     qkv        act   [B][T][C]           z, out  act/out [B][T][H_v][d_v]
 *     alpha,beta act   [B][T][H_v]         (beta already passed through its sigmoid)
 *     state      f32   [P][H_v][d_v][d_k]  S[i][j]: row i = value index, column j = key index
 *     conv_state f32   [P][3][C]           oldest row first
 *     conv_w     f32   [C][4]              tap 3 multiplies the current token
 *     norm_w     f32   [d_v] (shared by all heads);  A_log, dt_bias  f32 [H_v]
 *     capture->ssm   f32 [P][t_cap][H_v][d_v][d_k]  element t = state after token t
 *     capture->conv  f32 chain: [P][3 + t_cap][C]  the whole conv input window xext
 *                        tree:  [P][t_cap][3][C]   the 3-row conv state after each node
 *   (lucebox-hub internal.h, struct TargetCache, ssm_state / conv_state / ssm_intermediate /
 *   conv_input_cache comments; the pages give ggml shapes, the orientation here is a choice.)
 * - Every pointer is caller-owned device memory (the model does not own its cache: hf2q
 *   qwen35_target.rs, Qwen35DFlashTarget).  The library allocates nothing, keeps no device
 *   state, and only enqueues work on `stream` (a hipStream_t, NULL = the null stream); calls
 *   return before the GPU finishes.
 * - Batch entry b uses slot slot_ids[b] (device int32 [B]).  Slots within one call must be
 *   distinct.  Entries whose slot is outside [0, n_pool) are skipped by the kernels (nothing is
 *   read or written for them); GDN_F_CHECK_INDICES makes the host copy the index arrays back
 *   (synchronously) and fail with GDN_ERR_RANGE instead.  On a stream under capture that copy
 *   cannot be recorded: with the flag set such a call returns GDN_ERR_ARG and leaves the stream
 *   and its capture untouched.
 * - Return value: GDN_OK or an error code.  On error nothing has been enqueued and nothing is
 *   mutated; gdn_last_error() returns a thread-local description (lucebox-hub internal.h keeps
 *   one error sink, set_last_error).  GDN_ERR_HIP reports a failed launch.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum gdn_status {
    GDN_OK = 0,
    GDN_ERR_ARG = 1,    /* null pointer or inconsistent argument */
    GDN_ERR_SHAPE = 2,  /* unsupported or inconsistent dimensions */
    GDN_ERR_DTYPE = 3,  /* unsupported activation / output dtype */
    GDN_ERR_RANGE = 4,  /* slot, accepted index, token count or parent out of range */
    GDN_ERR_HIP = 5     /* the HIP runtime reported an error */
};

enum gdn_dtype { GDN_F32 = 0, GDN_BF16 = 1 };

enum gdn_capture_mode { GDN_CHAIN = 0, GDN_TREE = 1 };

/* SiLU after the conv on q, k and v; q and k scaled to unit length (x / sqrt(sum x^2 + 1e-6));
 * q scaled by d_k^-1/2.  Off by default: the recurrence as stated has none of these. */
#define GDN_F_QK_NORM_SILU 0x1u
/* Copy device index arrays (slot_ids, parent, rollback slots / indices) to the host and
 * validate them before launching.  Synchronises with `stream`. */
#define GDN_F_CHECK_INDICES 0x2u
/* Chain verify with capture (gdn_verify, gdn_verify_resume) leaves state[slot] and
 * conv_state[slot] untouched, as tree verify does: the state after the last token is capture
 * position n_tok-1 and its conv state window rows n_tok .. n_tok+2.  The caller commits a
 * position with gdn_rollback / gdn_rollback_batch, or passes it to the next round's
 * gdn_verify_resume, which reads it from the capture; so a round that accepts every token also
 * ends in a commit, unlike the pages' trim-0 early return (hf2q qwen35_target.rs, rollback_kv).
 * gdn_rollback_trim reads this flag from the capture's dims: with it, trim 0 commits position
 * n_tok - 1 instead of returning at once, so the capture descriptor of a deferred verify must
 * carry the flag.  A call of more than one launch (n_tok > 16) carries the state between its
 * launches through its own capture positions.  Without a capture it is GDN_ERR_ARG; other calls
 * ignore it. */
#define GDN_F_DEFER_COMMIT 0x4u

typedef struct gdn_dims {
    int32_t n_kh;      /* key heads H_k */
    int32_t n_vh;      /* value heads H_v, a multiple of H_k */
    int32_t d_k;       /* key head dim (64 or 128) */
    int32_t d_v;       /* value head dim, equal to d_k */
    int32_t d_conv;    /* conv kernel, must be 4 */
    int32_t n_pool;    /* P: slots in the state pool */
    int32_t act_dtype; /* gdn_dtype of qkv, z, alpha, beta */
    int32_t out_dtype; /* gdn_dtype of out */
    uint32_t flags;    /* GDN_F_* */
    float eps;         /* RMS-norm epsilon (1e-6 in the pages' model) */
} gdn_dims;

/* Persistent per-position capture written by a verify and read by rollback.  `state` and
 * `conv_state` name the buffers that rollback restores into.  lucebox-hub internal.h, struct
 * DeltaNetCapture: the capture lives in persistent cache buffers that outlive a call, not in
 * per-call scratch memory. */
typedef struct gdn_capture {
    gdn_dims dims;
    float *ssm;        /* [P][t_cap][H_v][d_v][d_k] */
    float *conv;       /* chain [P][3 + t_cap][C] or tree [P][t_cap][3][C] */
    float *state;      /* [P][H_v][d_v][d_k] */
    float *conv_state; /* [P][3][C] */
    int32_t t_cap;     /* capacity in positions (>= n_tok of every verify that writes it) */
    int32_t mode;      /* gdn_capture_mode */
} gdn_capture;

/*
 * Chain verify of n_tok tokens for n_batch slots (the K+1 drafted tokens of a speculative
 * round).  For each batch entry b and value head h: conv, gate, delta-rule update, readout and
 * norm/gate epilogue for every token, in order.  state[slot] and conv_state[slot] are advanced
 * to after the last token (so trim 0 needs no rollback: hf2q qwen35_target.rs, rollback_kv
 * returns at once for trim 0).  When `capture` is not NULL (mode GDN_CHAIN, t_cap >= n_tok), the
 * state after every token t goes to capture->ssm[slot][t] and the whole conv input window to
 * capture->conv[slot][0 .. 3+n_tok) (lucebox-hub internal.h, struct TargetCache: ssm_intermediate
 * and conv_input_cache).  capture == NULL is plain decode with no rollback support.
 *   qkv, z, alpha, beta: act_dtype;  out: out_dtype [n_batch][n_tok][H_v][d_v].
 *   1 <= n_tok;  1 <= n_batch <= n_pool.
 * Memory: with few heads in flight (n_batch * H_v * 4 <= 256, n_tok >= 3) the rows of each head
 * are split over several workgroups, which need a readout scratch: the first such call on a
 * stream allocates 4 MiB of device memory, kept for that stream until the process ends (calls on
 * different streams never share one).  Under stream capture no memory is allocated and no
 * stream's buffer is recorded (a recorded graph could be replayed on another stream while that
 * stream runs later calls): the capture gets the unsplit kernels, with the same results bit for
 * bit.  gdn_graph_create reserves a buffer for its own private capture stream and keeps it for the
 * graph's lifetime.
 */
int gdn_verify(const gdn_dims *dims, float *state, float *conv_state, const void *qkv,
               const void *z, const void *alpha, const void *beta, const float *A_log,
               const float *dt_bias, const float *conv_w, const float *norm_w,
               const gdn_capture *capture, void *out, int32_t n_tok, const int32_t *slot_ids,
               int32_t n_batch, void *stream);

/*
 * gdn_verify with the previous round's rollback folded into the state load.  For batch entry b
 * with r = resume_idx[b] >= 0, the first token starts from the state after capture position r of
 * `capture` and the conv state of window rows r+1 .. r+3: what gdn_rollback(capture, slot, r)
 * would have restored into the slot (hf2q qwen35_target.rs, rollback_kv: the state after the
 * accepted position; lucebox-hub internal.h, struct DeltaNetCapture: the state at offset
 * commit_n-1 and the conv slice from commit_n).  Entries with r < 0 start from state[slot] and
 * conv_state[slot], as gdn_verify does.  The same capture is then overwritten by this call's own
 * positions, in the same launch: a round's pending rollback costs no copy and no launch.  The
 * results, including state[slot] and conv_state[slot] after the last token, are bit-identical to
 * gdn_rollback (or gdn_rollback_batch) followed by gdn_verify.
 *   capture: required, mode GDN_CHAIN, t_cap >= n_tok; position r must hold what the previous
 *            verify of that slot wrote (r < that call's n_tok; the library cannot check this).
 *   resume_idx: device int32 [n_batch].  An entry with r >= t_cap is skipped: nothing of it is
 *            written.  With GDN_F_CHECK_INDICES it is GDN_ERR_RANGE before any launch.
 *   Every other argument as gdn_verify.  resume_idx or capture NULL -> GDN_ERR_ARG.
 */
int gdn_verify_resume(const gdn_dims *dims, float *state, float *conv_state, const void *qkv,
                      const void *z, const void *alpha, const void *beta, const float *A_log,
                      const float *dt_bias, const float *conv_w, const float *norm_w,
                      const gdn_capture *capture, void *out, int32_t n_tok,
                      const int32_t *slot_ids, const int32_t *resume_idx, int32_t n_batch,
                      void *stream);

/*
 * Tree verify: n_tok draft-tree nodes per batch entry, node i hanging off parent[b][i]
 * (device int32 [n_batch][n_tok]; -1 = starts from the committed state, else 0 <= parent < i;
 * node 0 is the root and must have parent -1).  lucebox-hub internal.h, QwenGraphInputs::
 * parent_ids (a non-null parent array selects tree verification); create_target_cache sizes the capture for
 * 1 + tree budget positions.  Node i's state is its parent's state advanced by node i's token;
 * its conv window runs along the ancestor path, filled from conv_state above the root.  Writes
 * out for every node, capture->ssm[slot][i] (state after node i) and capture->conv[slot][i]
 * (3-row conv state after node i; capture->mode must be GDN_TREE, t_cap >= n_tok).  state and
 * conv_state are NOT advanced: the caller commits a node with gdn_rollback.  Nodes with a
 * malformed parent are treated as children of the committed state unless GDN_F_CHECK_INDICES
 * is set (then GDN_ERR_RANGE).  n_tok is 1 .. 1024 (more: GDN_ERR_SHAPE).  Trees of more than 64
 * nodes run as consecutive launches of 64 nodes on `stream`; a node whose parent lies in an
 * earlier launch starts from that parent's capture, so the capture must not be written by
 * anything else while the call's launches run.
 */
int gdn_verify_tree(const gdn_dims *dims, const float *state, const float *conv_state,
                    const void *qkv, const void *z, const void *alpha, const void *beta,
                    const float *A_log, const float *dt_bias, const float *conv_w,
                    const float *norm_w, const int32_t *parent, const gdn_capture *capture,
                    void *out, int32_t n_tok, const int32_t *slot_ids, int32_t n_batch,
                    void *stream);

/*
 * Restore slot `slot` to the state after accepted position `accepted_idx` (host ints):
 *   capture->state[slot]      <- capture->ssm[slot][accepted_idx]            (bitwise copy)
 *   capture->conv_state[slot] <- capture->conv[slot][accepted_idx+1 .. +3]   (chain)
 *                                capture->conv[slot][accepted_idx]           (tree)
 * No other slot is read or written (hf2q qwen35_target.rs, rollback_kv: a per-slot rollback;
 * lucebox-hub internal.h, DeltaNetCapture: offset (commit_n-1) and conv slice
 * [commit_n .. commit_n+kernel-2]).  Errors: slot not in [0, n_pool) or accepted_idx not in
 * [0, t_cap) -> GDN_ERR_RANGE (the pages skip silently; here the caller hears of it).
 */
int gdn_rollback(const gdn_capture *capture, int32_t slot, int32_t accepted_idx, void *stream);

/*
 * Batched rollback of n entries in one launch: slots and accepted_idx are device int32 [n];
 * entry i does what gdn_rollback(capture, slots[i], accepted_idx[i]) does.  The pages roll back
 * one slot per call, each slot from its own accepted position (hf2q qwen35_target.rs, rollback_kv
 * and rollback_la_to, per SlotId); the slots of a verify batch are independent, so their copies
 * share one launch.  Entries with an out-of-range slot or index are skipped (GDN_F_CHECK_INDICES
 * in capture->dims.flags: validated on the host, GDN_ERR_RANGE).  Slots must be distinct.
 * n == 0 is a no-op; n outside [0, min(n_pool, 65535)] is GDN_ERR_RANGE.
 */
int gdn_rollback_batch(const gdn_capture *capture, const int32_t *slots,
                       const int32_t *accepted_idx, int32_t n, void *stream);

/*
 * The pages' trim form (hf2q qwen35_target.rs, rollback_kv): n_tok positions were verified,
 * the last `trim` are rejected.  trim == 0 -> GDN_OK with nothing enqueued, because the verify
 * already left the state after its last token; but when capture->dims.flags has
 * GDN_F_DEFER_COMMIT that verify left the state in the capture, and trim 0 is
 * gdn_rollback(capture, slot, n_tok - 1).  trim >= n_tok -> GDN_ERR_RANGE; else
 * gdn_rollback(capture, slot, n_tok - 1 - trim).  n_tok outside [1, t_cap], a negative trim or a
 * slot outside [0, n_pool) -> GDN_ERR_RANGE.  Chain captures only: a tree's node indices are not
 * positions along one path (a GDN_TREE capture -> GDN_ERR_ARG; roll a tree back with gdn_rollback
 * at the accepted node).
 */
int gdn_rollback_trim(const gdn_capture *capture, int32_t slot, int32_t trim, int32_t n_tok,
                      void *stream);

/*
 * Chunked prefill of n_tok tokens into slot `slot` (no capture: a prefill-only cache skips the
 * rollback tensors, lucebox-hub internal.h, create_target_cache prefill_only).  Same result as
 * gdn_verify with capture == NULL, computed in chunks of 64 tokens in the WY/UT form with the
 * dense intra-chunk products on MFMA.  workspace: device memory of at least
 * gdn_prefill_workspace_bytes(dims, n_tok) bytes (per-chunk operands and the fp32 readout; its
 * contents need no initialisation and are garbage afterwards).
 *   qkv [n_tok][C], z and out [n_tok][H_v][d_v], alpha and beta [n_tok][H_v].
 * state, conv_state, conv_w, qkv, z, out, norm_w and workspace must be 16-byte aligned
 * (GDN_ERR_ARG).
 */
int gdn_prefill(const gdn_dims *dims, float *state, float *conv_state, const void *qkv,
                const void *z, const void *alpha, const void *beta, const float *A_log,
                const float *dt_bias, const float *conv_w, const float *norm_w, void *out,
                int32_t n_tok, int32_t slot, void *workspace, size_t ws_bytes, void *stream);

/*
 * gdn_prefill for callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  Same arguments as gdn_prefill without
 * the workspace, same results: the workspace is a static device array of
 * GDN_NOALLOC_SCRATCH_BYTES inside the library (one per GPU, held from the first call on that GPU
 * until the process ends; looked up with hipGetSymbolAddress on that first call, which is the
 * only call that can fail with GDN_ERR_HIP before launching).  The call runs as consecutive
 * pieces of the most whole 64-token chunks whose workspace fits the array (the state carries over
 * between pieces as between two gdn_prefill calls); dims whose single chunk needs more than the
 * array are GDN_ERR_SHAPE.  No hipMalloc, hipFree or allocating library routine is called.  Every
 * call on one GPU shares that GPU's array: calls that overlap on one GPU (on different streams,
 * or from different host threads without ordering) race and must not be issued.  Every other
 * error as gdn_prefill; a launch failure (GDN_ERR_HIP) may leave earlier pieces enqueued.
 */
#define GDN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int gdn_prefill_noalloc(const gdn_dims *dims, float *state, float *conv_state, const void *qkv,
                        const void *z, const void *alpha, const void *beta, const float *A_log,
                        const float *dt_bias, const float *conv_w, const float *norm_w, void *out,
                        int32_t n_tok, int32_t slot, void *stream);

/* Workspace bytes gdn_prefill needs for n_tok tokens (0 on invalid dims or n_tok < 1).  The
 * pages' prefill keeps its per-call intermediates in the compute graph's own buffers, apart from
 * the persistent cache (lucebox-hub internal.h, create_target_cache: a prefill-only cache holds no
 * rollback tensors); here the caller owns that memory and sizes it with this call. */
size_t gdn_prefill_workspace_bytes(const gdn_dims *dims, int32_t n_tok);

/* Bytes of capture->ssm for t_cap positions; *conv_bytes (if not NULL) receives the bytes of
 * capture->conv for the mode (0 on invalid dims, t_cap < 1 or an unknown mode).  The pages size
 * the capture by the most positions one verify writes (lucebox-hub internal.h, struct TargetCache:
 * ssm_intermediate [S_v, S_v, H_v, max_q_len] and conv_input_cache [(kernel-1) + max_q_len,
 * conv_channels] per layer; the create_target_cache comment sets that length from
 * max_verify_tokens, at least 1 + the tree budget in tree mode): chain P * t_cap * H_v * d_v * d_k
 * and P * (3 + t_cap) * C floats, tree P * t_cap * 3 * C for the conv. */
size_t gdn_capture_bytes(const gdn_dims *dims, int32_t t_cap, int32_t mode, size_t *conv_bytes);

/* Zero the recurrent state and conv state of one slot (lucebox-hub internal.h,
 * reset_recurrent_state: zero SSM + conv state between requests). */
int gdn_reset(const gdn_dims *dims, float *state, float *conv_state, int32_t slot,
              void *stream);

/*
 * Snapshot-and-replay rollback, the alternative to the per-position capture.  lucebox-hub
 * internal.h, snapshot_ssm_state / restore_ssm_state: the recurrent and conv state are copied to
 * and from snapshot tensors (TargetCache ssm_state_snap, conv_state_snap) shaped like the live
 * ones.  A spec-decode round then runs: gdn_snapshot, gdn_verify with capture == NULL over the
 * K+1 drafted tokens, and only if some are rejected gdn_restore followed by gdn_verify (again
 * without capture) over the accepted tokens.  It moves the state about three times instead of
 * writing K+1 captures, at the price of a second pass on rejection.
 *
 * gdn_snapshot copies, for each of the n slots in `slots` (device int32 [n], distinct), the slot's
 * state [H_v][d_v][d_k] and conv state [3][C] from state / conv_state into snap_state / snap_conv;
 * gdn_restore copies them back.  The snapshot buffers have the pool layout of state and conv_state
 * ([P][H_v][d_v][d_k] and [P][3][C] fp32, caller-owned, 16-byte aligned); only the listed slots
 * are read or written.  Bitwise copies, stream-ordered.  n == 0 is a no-op; n outside
 * [0, min(n_pool, 65535)] is GDN_ERR_RANGE; NULL or misaligned buffers GDN_ERR_ARG.  Slots outside
 * [0, n_pool) are skipped, or rejected with GDN_ERR_RANGE under GDN_F_CHECK_INDICES (which also
 * rejects repeated slots).
 */
int gdn_snapshot(const gdn_dims *dims, const float *state, const float *conv_state, float *snap_state,
                 float *snap_conv, const int32_t *slots, int32_t n, void *stream);
int gdn_restore(const gdn_dims *dims, float *state, float *conv_state, const float *snap_state,
                const float *snap_conv, const int32_t *slots, int32_t n, void *stream);

/*
 * Rollback of every GDN layer of a model in one launch.  The pages keep one capture per
 * delta-net layer (lucebox-hub internal.h, struct TargetCache: ssm_intermediate and
 * conv_input_cache, one each per layer) and a slot's rollback restores all of them (hf2q
 * qwen35_target.rs, rollback_kv: the LA-state rollback covers the model's linear-attention
 * layers for that slot).
 *   layers: host array of n_layers capture descriptors, one per layer, all with equal dims,
 *     t_cap and mode; no two may share a state or conv_state buffer.  Read during the call only.
 *   slots, accepted_idx: device int32 [n], shared by every layer (a slot accepts the same
 *     drafted tokens in every layer).
 * For every layer l the result is that of gdn_rollback_batch(&layers[l], slots, accepted_idx,
 * n): bitwise copies, stream-ordered, entries with an out-of-range slot or index skipped (under
 * GDN_F_CHECK_INDICES in layers[0].dims.flags: GDN_ERR_RANGE).  Up to 64 layers go into one
 * launch; more take one launch per 64.  n == 0 is a no-op; n outside [0, min(n_pool, 65535)] or
 * n_layers < 1 is GDN_ERR_RANGE; NULL layers, a bad descriptor, descriptors that differ in dims,
 * t_cap or mode, or a shared state buffer are GDN_ERR_ARG.
 */
int gdn_rollback_layers(const gdn_capture *layers, int32_t n_layers, const int32_t *slots,
                        const int32_t *accepted_idx, int32_t n, void *stream);

/*
 * A whole GDN spec-decode step recorded once as a HIP graph and replayed with one launch.  The
 * pages replay a recorded graph per step to cut launch overhead (lucebox dflash_draft_kv.h: the
 * draft's CUDA graph is replayed each step; lucebox-hub internal.h, the note on the number of
 * graph launches per step) and keep one capture per delta-net layer (struct TargetCache).
 *
 * gdn_layer names one layer's buffers, with the meaning and layout of the gdn_verify arguments of
 * the same names; cap_ssm / cap_conv form that layer's chain capture of t_cap positions, restored
 * into state / conv_state.
 */
typedef struct gdn_layer {
    float *state;
    float *conv_state;
    const void *qkv, *z, *alpha, *beta;
    const float *A_log, *dt_bias, *conv_w, *norm_w;
    float *cap_ssm;
    float *cap_conv;
    void *out;
} gdn_layer;

#define GDN_GRAPH_VERIFY 0x1u   /* gdn_verify of every layer, in layer order, capture on */
#define GDN_GRAPH_ROLLBACK 0x2u /* then gdn_rollback_layers of every layer */

typedef struct gdn_graph gdn_graph; /* opaque; owned by the caller between create and destroy */

/*
 * Record the phases in `phases` (GDN_GRAPH_* bits, at least one) for n_layers layers, n_tok
 * tokens and the n_batch slots in slot_ids (device int32 [n_batch]); the rollback phase restores
 * the slots of slot_ids to accepted_idx (device int32 [n_batch]).  Every argument is checked as
 * the corresponding gdn_verify / gdn_rollback_layers call checks it, once, here.  The graph keeps
 * the pointers and sizes given now and reads what they point at when it runs, so between
 * launches the caller rewrites activations, slot ids and accepted indices in place.  The layer
 * array is read during the call only.  GDN_F_CHECK_INDICES is rejected (GDN_ERR_ARG): its host
 * copy cannot be recorded.  Recording uses a private stream and allocates the graph; on error
 * *graph is NULL and nothing is left allocated.
 */
int gdn_graph_create(const gdn_dims *dims, const gdn_layer *layers, int32_t n_layers, int32_t t_cap,
                     int32_t n_tok, const int32_t *slot_ids, int32_t n_batch,
                     const int32_t *accepted_idx, uint32_t phases, gdn_graph **graph);
/* Enqueue one replay of the recorded step on `stream`.  Replays on one graph must not overlap. */
int gdn_graph_launch(const gdn_graph *graph, void *stream);
/* Free the graph (NULL is a no-op).  Pending replays finish first. */
int gdn_graph_destroy(gdn_graph *graph);

/*
 * The GDN block's projections on MFMA: y = x W^T with x [M][K] and W [N][K] bf16 (row-major; W
 * holds one output feature per row, input index fastest), fp32 accumulation.  lucebox-hub
 * internal.h, struct TargetLayer: wqkv (fused q / k / v), wqkv_gate (z), ssm_beta, ssm_alpha
 * (per-token projections) and ssm_out (output projection); the four input projections are one
 * call over their concatenated weights, split by gdn_out_seg.
 *
 * segs[0 .. n_segs) cut the product's columns into consecutive ranges [n0, n1) (segs[0].n0 = 0,
 * each n0 the previous n1, the last n1 = N); column n of segment s, row m, is stored at
 * ptr[m * ld + (n - n0)] as dtype (GDN_BF16, round to nearest even, or GDN_F32), through
 * 1 / (1 + e^-v) when sigmoid is nonzero.  Errors: NULL or misaligned x / W (16 bytes) or a NULL
 * ptr -> GDN_ERR_ARG; M, N < 1 or K not a positive multiple of 64 -> GDN_ERR_SHAPE; n_segs
 * outside [1, 4], ranges that do not tile [0, N), ld < n1 - n0 -> GDN_ERR_ARG; bad dtype ->
 * GDN_ERR_DTYPE.
 */
typedef struct gdn_out_seg {
    int32_t n0, n1; /* product columns [n0, n1) */
    int32_t ld;     /* destination row stride in elements (>= n1 - n0) */
    int32_t dtype;  /* GDN_BF16 or GDN_F32 */
    int32_t sigmoid;
    void *ptr;
} gdn_out_seg;
int gdn_linear(const void *x, const void *w, int32_t M, int32_t N, int32_t K, const gdn_out_seg *segs,
               int32_t n_segs, void *stream);

/* Thread-local description of the last error of this thread ("" after success).  The pages'
 * header keeps one error-reporting channel that its loaders and graph builders write to, with
 * calls returning failure and leaving the message there (lucebox-hub internal.h, set_last_error);
 * every entry point here returns a status code and leaves its message for this call. */
const char *gdn_last_error(void);

/* Library version string. */
const char *gdn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
