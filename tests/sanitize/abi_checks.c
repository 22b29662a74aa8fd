/* Host-side validation of every entry point of gdn.h, for a build of the library's host code under
 * AddressSanitizer and UndefinedBehaviorSanitizer (device code is not built: nothing here reaches a
 * launch).  Each call passes a bad argument and must return its documented code without touching
 * memory it does not own; the fake pointers below are never dereferenced.  Exit status 0 = all
 * checks passed; the sanitizers abort on any memory or UB error. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "gdn.h"

static int failures = 0;
#define CHECK(call, want)                                                                              \
    do {                                                                                               \
        int got_ = (call);                                                                             \
        if (got_ != (want)) {                                                                          \
            fprintf(stderr, "%s:%d: %s returned %d, expected %d (%s)\n", __FILE__, __LINE__, #call, got_, \
                    (int)(want), gdn_last_error());                                                    \
            ++failures;                                                                                \
        }                                                                                              \
    } while (0)

int main(void)
{
    void *F = (void *)(uintptr_t)0x1000; /* aligned, never dereferenced */
    void *MIS = (void *)(uintptr_t)0x1008;
    gdn_dims d;
    memset(&d, 0, sizeof d);
    d.n_kh = 16; d.n_vh = 32; d.d_k = 128; d.d_v = 128; d.d_conv = 4; d.n_pool = 4;
    d.act_dtype = GDN_BF16; d.out_dtype = GDN_BF16; d.flags = 0; d.eps = 1e-6f;

    /* verify */
    gdn_dims bad = d; bad.d_conv = 3;
    CHECK(gdn_verify(&bad, F, F, F, F, F, F, F, F, F, F, NULL, F, 4, F, 1, NULL), GDN_ERR_SHAPE);
    bad = d; bad.act_dtype = 9;
    CHECK(gdn_verify(&bad, F, F, F, F, F, F, F, F, F, F, NULL, F, 4, F, 1, NULL), GDN_ERR_DTYPE);
    CHECK(gdn_verify(NULL, F, F, F, F, F, F, F, F, F, F, NULL, F, 4, F, 1, NULL), GDN_ERR_ARG);
    CHECK(gdn_verify(&d, NULL, F, F, F, F, F, F, F, F, F, NULL, F, 4, F, 1, NULL), GDN_ERR_ARG);
    CHECK(gdn_verify(&d, MIS, F, F, F, F, F, F, F, F, F, NULL, F, 4, F, 1, NULL), GDN_ERR_ARG);
    CHECK(gdn_verify(&d, F, F, F, F, F, F, F, F, F, F, NULL, F, 0, F, 1, NULL), GDN_ERR_RANGE);
    CHECK(gdn_verify(&d, F, F, F, F, F, F, F, F, F, F, NULL, F, 4, F, 5, NULL), GDN_ERR_RANGE);
    gdn_capture cap;
    memset(&cap, 0, sizeof cap);
    cap.dims = d; cap.ssm = F; cap.conv = F; cap.state = F; cap.conv_state = F; cap.t_cap = 2; cap.mode = GDN_CHAIN;
    CHECK(gdn_verify(&d, F, F, F, F, F, F, F, F, F, F, &cap, F, 4, F, 1, NULL), GDN_ERR_RANGE); /* t_cap < n_tok */
    cap.t_cap = 16; cap.mode = GDN_TREE;
    CHECK(gdn_verify(&d, F, F, F, F, F, F, F, F, F, F, &cap, F, 4, F, 1, NULL), GDN_ERR_ARG); /* wrong mode */
    /* a deferred commit needs the capture */
    gdn_dims defer = d; defer.flags = GDN_F_DEFER_COMMIT;
    CHECK(gdn_verify(&defer, F, F, F, F, F, F, F, F, F, F, NULL, F, 4, F, 1, NULL), GDN_ERR_ARG);
    /* verify resuming from capture positions */
    cap.t_cap = 16; cap.mode = GDN_CHAIN;
    CHECK(gdn_verify_resume(&d, F, F, F, F, F, F, F, F, F, F, &cap, F, 4, F, NULL, 1, NULL), GDN_ERR_ARG);
    CHECK(gdn_verify_resume(&d, F, F, F, F, F, F, F, F, F, F, NULL, F, 4, F, F, 1, NULL), GDN_ERR_ARG);
    CHECK(gdn_verify_resume(&d, F, F, F, F, F, F, F, F, F, F, &cap, F, 0, F, F, 1, NULL), GDN_ERR_RANGE);
    CHECK(gdn_verify_resume(&d, F, F, F, F, F, F, F, F, F, F, &cap, F, 4, F, F, 5, NULL), GDN_ERR_RANGE);
    cap.mode = GDN_TREE;
    CHECK(gdn_verify_resume(&d, F, F, F, F, F, F, F, F, F, F, &cap, F, 4, F, F, 1, NULL), GDN_ERR_ARG);
    /* tree */
    CHECK(gdn_verify_tree(&d, F, F, F, F, F, F, F, F, F, F, NULL, &cap, F, 4, F, 1, NULL), GDN_ERR_ARG);
    CHECK(gdn_verify_tree(&d, F, F, F, F, F, F, F, F, F, F, F, &cap, F, 0, F, 1, NULL), GDN_ERR_RANGE);
    /* rollback */
    cap.mode = GDN_CHAIN;
    CHECK(gdn_rollback(NULL, 0, 0, NULL), GDN_ERR_ARG);
    CHECK(gdn_rollback(&cap, 4, 0, NULL), GDN_ERR_RANGE);
    CHECK(gdn_rollback(&cap, 0, 16, NULL), GDN_ERR_RANGE);
    CHECK(gdn_rollback(&cap, -1, 0, NULL), GDN_ERR_RANGE);
    CHECK(gdn_rollback_batch(&cap, NULL, NULL, 0, NULL), GDN_OK);
    CHECK(gdn_rollback_batch(&cap, NULL, NULL, 2, NULL), GDN_ERR_ARG);
    CHECK(gdn_rollback_batch(&cap, F, F, 5, NULL), GDN_ERR_RANGE);
    CHECK(gdn_rollback_trim(&cap, 0, 0, 16, NULL), GDN_OK);
    CHECK(gdn_rollback_trim(&cap, 0, 16, 16, NULL), GDN_ERR_RANGE);
    CHECK(gdn_rollback_trim(&cap, 0, 3, 17, NULL), GDN_ERR_RANGE);
    cap.mode = GDN_TREE;
    CHECK(gdn_rollback_trim(&cap, 0, 3, 16, NULL), GDN_ERR_ARG); /* trim counts chain positions */
    cap.mode = GDN_CHAIN;
    gdn_capture two[2];
    two[0] = cap; two[1] = cap;
    CHECK(gdn_rollback_layers(two, 2, F, F, 1, NULL), GDN_ERR_ARG); /* shared state buffer */
    two[0].conv_state = (void *)(uintptr_t)0x4000;
    two[1].state = (void *)(uintptr_t)0x2000; two[1].conv_state = (void *)(uintptr_t)0x3000;
    CHECK(gdn_rollback_layers(two, 2, NULL, NULL, 0, NULL), GDN_OK);
    CHECK(gdn_rollback_layers(two, 0, F, F, 1, NULL), GDN_ERR_RANGE);
    two[1].t_cap = 8;
    CHECK(gdn_rollback_layers(two, 2, F, F, 1, NULL), GDN_ERR_ARG);
    /* prefill */
    CHECK(gdn_prefill(&d, F, F, F, F, F, F, F, F, F, F, F, 0, 0, F, (size_t)1 << 40, NULL), GDN_ERR_RANGE);
    CHECK(gdn_prefill(&d, F, F, F, F, F, F, F, F, F, F, F, 64, 4, F, (size_t)1 << 40, NULL), GDN_ERR_RANGE);
    CHECK(gdn_prefill(&d, F, F, F, F, F, F, F, F, F, F, F, 64, 0, F, 16, NULL), GDN_ERR_ARG);
    CHECK(gdn_prefill(&d, F, F, F, F, F, F, F, F, F, F, F, 64, 0, NULL, (size_t)1 << 40, NULL), GDN_ERR_ARG);
    /* prefill without a workspace argument: the same validation, before the scratch is looked up */
    CHECK(gdn_prefill_noalloc(&d, F, F, F, F, F, F, F, F, F, F, F, 0, 0, NULL), GDN_ERR_RANGE);
    CHECK(gdn_prefill_noalloc(&d, F, F, F, F, F, F, F, F, F, F, F, 64, 4, NULL), GDN_ERR_RANGE);
    CHECK(gdn_prefill_noalloc(&d, F, F, F, F, F, F, F, F, F, F, NULL, 64, 0, NULL), GDN_ERR_ARG);
    CHECK(gdn_prefill_noalloc(&d, MIS, F, F, F, F, F, F, F, F, F, F, 64, 0, NULL), GDN_ERR_ARG);
    CHECK(gdn_prefill_noalloc(NULL, F, F, F, F, F, F, F, F, F, F, F, 64, 0, NULL), GDN_ERR_ARG);
    if (gdn_prefill_workspace_bytes(&d, 0) != 0) { fprintf(stderr, "workspace bytes for 0 tokens\n"); ++failures; }
    if (gdn_prefill_workspace_bytes(&d, 8192) != 373293056u) { fprintf(stderr, "workspace bytes at 8192\n"); ++failures; }
    /* sizes, reset, snapshot */
    size_t cb = 1;
    if (gdn_capture_bytes(&bad, 16, GDN_CHAIN, &cb) != 0 || cb != 0) { fprintf(stderr, "capture bytes of bad dims\n"); ++failures; }
    CHECK(gdn_reset(&d, F, F, 4, NULL), GDN_ERR_RANGE);
    CHECK(gdn_reset(&d, MIS, F, 0, NULL), GDN_ERR_ARG);
    CHECK(gdn_snapshot(&d, F, F, F, F, NULL, 0, NULL), GDN_OK);
    CHECK(gdn_snapshot(&d, F, F, F, F, F, 5, NULL), GDN_ERR_RANGE);
    CHECK(gdn_restore(&d, F, F, F, F, NULL, 2, NULL), GDN_ERR_ARG);
    /* graph */
    gdn_graph *g = (gdn_graph *)F;
    gdn_layer lay;
    memset(&lay, 0, sizeof lay);
    CHECK(gdn_graph_create(&d, &lay, 1, 16, 16, F, 1, F, GDN_GRAPH_VERIFY, &g), GDN_ERR_ARG); /* NULL buffers */
    if (g != NULL) { fprintf(stderr, "graph handle not cleared on error\n"); ++failures; }
    CHECK(gdn_graph_create(&d, &lay, 0, 16, 16, F, 1, F, GDN_GRAPH_VERIFY, &g), GDN_ERR_RANGE);
    CHECK(gdn_graph_create(&d, &lay, 1, 16, 16, F, 1, F, 0, &g), GDN_ERR_ARG);
    CHECK(gdn_graph_launch(NULL, NULL), GDN_ERR_ARG);
    CHECK(gdn_graph_destroy(NULL), GDN_OK);
    /* linear */
    gdn_out_seg seg[2];
    memset(seg, 0, sizeof seg);
    seg[0].n0 = 0; seg[0].n1 = 100; seg[0].ld = 100; seg[0].dtype = GDN_BF16; seg[0].ptr = F;
    seg[1].n0 = 100; seg[1].n1 = 164; seg[1].ld = 64; seg[1].dtype = GDN_F32; seg[1].sigmoid = 1; seg[1].ptr = F;
    CHECK(gdn_linear(NULL, F, 8, 164, 128, seg, 2, NULL), GDN_ERR_ARG);
    CHECK(gdn_linear(F, F, 8, 164, 96, seg, 2, NULL), GDN_ERR_SHAPE);
    CHECK(gdn_linear(F, F, 8, 200, 128, seg, 2, NULL), GDN_ERR_ARG);
    CHECK(gdn_linear(F, F, 8, 164, 128, seg, 5, NULL), GDN_ERR_ARG);
    seg[1].dtype = 7;
    CHECK(gdn_linear(F, F, 8, 164, 128, seg, 2, NULL), GDN_ERR_DTYPE);
    /* the message of the last failure is a valid C string */
    if (strlen(gdn_last_error()) == 0) { fprintf(stderr, "empty last error\n"); ++failures; }
    if (strstr(gdn_version(), "gfx950") == NULL) { fprintf(stderr, "version\n"); ++failures; }
    printf("abi_checks: %d failures\n", failures);
    return failures != 0;
}
