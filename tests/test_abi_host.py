"""The C ABI on the host: the library loads, exports every symbol gdn.h declares, and rejects
bad arguments before touching the GPU (no compute call is made here)."""

import ctypes
import os
import re

import pytest

from gated_deltanet_linear_verify_amd import gdn
from gated_deltanet_linear_verify_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib_or_skip():
    if not os.path.exists(gdn.LIB_PATH):
        pytest.skip("libgdn.so not built")
    return gdn.lib()


def test_header_declarations_are_all_exported():
    L = _lib_or_skip()
    hdr = open(os.path.join(ROOT, "include", "gdn.h")).read()
    declared = set(re.findall(r"\b(gdn_[a-z_]+)\s*\(", hdr))
    assert declared == set(gdn.EXPORTS), declared ^ set(gdn.EXPORTS)
    for name in declared:
        assert hasattr(L, name), name


def test_version_and_empty_error():
    _lib_or_skip()
    assert "gfx950" in gdn.version()


FAKE = ctypes.c_void_p(0x1000)  # an aligned non-null address never dereferenced (rejected first)


def _dims(**kw):
    d = gdn.make_dims(W.SINGLE_SLOT_VERIFY)
    for k, v in kw.items():
        setattr(d, k, v)
    return d


@pytest.mark.parametrize("kw,code", [
    ({"d_conv": 3}, gdn.GDN_ERR_SHAPE),
    ({"d_k": 96, "d_v": 96}, gdn.GDN_ERR_SHAPE),
    ({"d_v": 64}, gdn.GDN_ERR_SHAPE),
    ({"n_vh": 24, "n_kh": 16}, gdn.GDN_ERR_SHAPE),
    ({"n_vh": 80, "n_kh": 16}, gdn.GDN_ERR_SHAPE),
    ({"n_pool": 0}, gdn.GDN_ERR_SHAPE),
    ({"act_dtype": 7}, gdn.GDN_ERR_DTYPE),
    ({"flags": 0x100}, gdn.GDN_ERR_ARG),
    ({"eps": -1.0}, gdn.GDN_ERR_ARG),
])
def test_verify_rejects_bad_dims(kw, code):
    L = _lib_or_skip()
    d = _dims(**kw)
    rc = L.gdn_verify(ctypes.byref(d), *([FAKE] * 10), None, FAKE, 4, FAKE, 1, None)
    assert rc == code, gdn.last_error()
    assert gdn.last_error()


def test_verify_rejects_null_and_range_before_launch():
    L = _lib_or_skip()
    d = _dims()
    args = [FAKE] * 10
    assert L.gdn_verify(ctypes.byref(d), *args, None, None, 4, FAKE, 1, None) == gdn.GDN_ERR_ARG
    assert L.gdn_verify(ctypes.byref(d), *args, None, FAKE, 0, FAKE, 1, None) == gdn.GDN_ERR_RANGE
    assert L.gdn_verify(ctypes.byref(d), *args, None, FAKE, 4, FAKE, 2, None) == gdn.GDN_ERR_RANGE
    mis = ctypes.c_void_p(0x1004)
    assert L.gdn_verify(ctypes.byref(d), mis, *args[1:], None, FAKE, 4, FAKE, 1, None) == gdn.GDN_ERR_ARG
    # capture too small for n_tok
    cap = gdn.gdn_capture(d, 0x1000, 0x1000, 0x1000, 0x1000, 3, gdn.GDN_CHAIN)
    assert L.gdn_verify(ctypes.byref(d), *args, ctypes.byref(cap), FAKE, 4, FAKE, 1, None) == gdn.GDN_ERR_RANGE
    cap = gdn.gdn_capture(d, 0x1000, 0x1000, 0x1000, 0x1000, 16, gdn.GDN_TREE)
    assert L.gdn_verify(ctypes.byref(d), *args, ctypes.byref(cap), FAKE, 4, FAKE, 1, None) == gdn.GDN_ERR_ARG


def test_verify_resume_validation():
    L = _lib_or_skip()
    d = _dims()
    args = [FAKE] * 10
    cap = gdn.gdn_capture(d, 0x1000, 0x1000, 0x1000, 0x1000, 16, gdn.GDN_CHAIN)
    # resume_idx and capture are required
    assert L.gdn_verify_resume(ctypes.byref(d), *args, ctypes.byref(cap), FAKE, 4, FAKE, None, 1,
                               None) == gdn.GDN_ERR_ARG
    assert L.gdn_verify_resume(ctypes.byref(d), *args, None, FAKE, 4, FAKE, FAKE, 1, None) == gdn.GDN_ERR_ARG
    # the rest is gdn_verify's validation
    assert L.gdn_verify_resume(ctypes.byref(d), *args, ctypes.byref(cap), FAKE, 0, FAKE, FAKE, 1,
                               None) == gdn.GDN_ERR_RANGE
    assert L.gdn_verify_resume(ctypes.byref(d), *args, ctypes.byref(cap), FAKE, 4, FAKE, FAKE, 2,
                               None) == gdn.GDN_ERR_RANGE
    small = gdn.gdn_capture(d, 0x1000, 0x1000, 0x1000, 0x1000, 3, gdn.GDN_CHAIN)
    assert L.gdn_verify_resume(ctypes.byref(d), *args, ctypes.byref(small), FAKE, 4, FAKE, FAKE, 1,
                               None) == gdn.GDN_ERR_RANGE
    tree = gdn.gdn_capture(d, 0x1000, 0x1000, 0x1000, 0x1000, 16, gdn.GDN_TREE)
    assert L.gdn_verify_resume(ctypes.byref(d), *args, ctypes.byref(tree), FAKE, 4, FAKE, FAKE, 1,
                               None) == gdn.GDN_ERR_ARG
    assert "resume" in gdn.last_error() or "mode" in gdn.last_error()
    # a deferred commit keeps the state in the capture, so it needs one
    dd = _dims(flags=gdn.GDN_F_DEFER_COMMIT)
    assert L.gdn_verify(ctypes.byref(dd), *args, None, FAKE, 4, FAKE, 1, None) == gdn.GDN_ERR_ARG
    assert "DEFER" in gdn.last_error()


def test_rollback_validation():
    L = _lib_or_skip()
    d = _dims(n_pool=4)
    cap = gdn.gdn_capture(d, 0x1000, 0x1000, 0x1000, 0x1000, 16, gdn.GDN_CHAIN)
    assert L.gdn_rollback(ctypes.byref(cap), 4, 0, None) == gdn.GDN_ERR_RANGE
    assert L.gdn_rollback(ctypes.byref(cap), -1, 0, None) == gdn.GDN_ERR_RANGE
    assert L.gdn_rollback(ctypes.byref(cap), 0, 16, None) == gdn.GDN_ERR_RANGE
    assert L.gdn_rollback(ctypes.byref(cap), 0, -1, None) == gdn.GDN_ERR_RANGE
    assert L.gdn_rollback(None, 0, 0, None) == gdn.GDN_ERR_ARG
    # trim form: trim 0 is a no-op that enqueues nothing; trim >= n_tok is a range error
    assert L.gdn_rollback_trim(ctypes.byref(cap), 0, 0, 16, None) == gdn.GDN_OK
    assert L.gdn_rollback_trim(ctypes.byref(cap), 0, 16, 16, None) == gdn.GDN_ERR_RANGE
    assert L.gdn_rollback_trim(ctypes.byref(cap), 0, 3, 17, None) == gdn.GDN_ERR_RANGE
    # the trim form counts positions along a chain; a tree capture is rejected
    tcap = gdn.gdn_capture(d, 0x1000, 0x1000, 0x1000, 0x1000, 16, gdn.GDN_TREE)
    assert L.gdn_rollback_trim(ctypes.byref(tcap), 0, 3, 16, None) == gdn.GDN_ERR_ARG
    assert "CHAIN" in gdn.last_error()
    assert L.gdn_rollback_batch(ctypes.byref(cap), None, None, 0, None) == gdn.GDN_OK
    assert L.gdn_rollback_batch(ctypes.byref(cap), None, None, 2, None) == gdn.GDN_ERR_ARG
    assert L.gdn_rollback_batch(ctypes.byref(cap), FAKE, FAKE, 5, None) == gdn.GDN_ERR_RANGE
    bad = gdn.gdn_capture(d, 0x1000, 0x1000, 0x1000, 0x1000, 16, 5)
    assert L.gdn_rollback(ctypes.byref(bad), 0, 0, None) == gdn.GDN_ERR_ARG


def test_capture_bytes_match_layout():
    _lib_or_skip()
    s = W.MULTI_SLOT_VERIFY
    d = gdn.make_dims(s)
    ssm, conv = gdn.capture_bytes(d, 16, gdn.GDN_CHAIN)
    assert ssm == 4 * 64 * 16 * 32 * 128 * 128 == 2 * 1024 ** 3
    assert conv == 4 * 64 * (3 + 16) * 8192
    ssm_t, conv_t = gdn.capture_bytes(d, 64, gdn.GDN_TREE)
    assert conv_t == 4 * 64 * 64 * 3 * 8192
    assert gdn.capture_bytes(d, 0, gdn.GDN_CHAIN) == (0, 0)


def test_prefill_validation():
    """gdn_prefill rejects bad arguments before any launch.  The workspace holds, per 64-token
    chunk, the fp32 readout (64 H_v d), q and k per key head (2 H_k 64 d), T and P per value head
    (2 H_v x the 3072 entries of a 64 x 64 lower-triangular matrix outside its zero upper-right
    32 x 32 block) and a 256-float gate record per value head."""
    L = _lib_or_skip()
    d = gdn.make_dims(W.CHUNKED_PREFILL)
    per_chunk = 64 * 32 * 128 + 2 * 16 * 64 * 128 + 2 * 32 * (64 * 64 - 32 * 32) + 32 * 256
    assert L.gdn_prefill_workspace_bytes(ctypes.byref(d), 8192) == 4 * 128 * per_chunk == 373_293_056
    assert L.gdn_prefill_workspace_bytes(ctypes.byref(d), 65) == 4 * 2 * per_chunk  # whole chunks
    assert L.gdn_prefill_workspace_bytes(ctypes.byref(d), 0) == 0
    big = 1 << 40
    args = [FAKE] * 11  # state .. out

    def call(dims, n_tok=64, slot=0, ws=FAKE, ws_bytes=big, a=args):
        return L.gdn_prefill(ctypes.byref(dims), *a, n_tok, slot, ws, ws_bytes, None)

    assert call(d, n_tok=0) == gdn.GDN_ERR_RANGE
    assert call(d, slot=1) == gdn.GDN_ERR_RANGE
    assert call(d, slot=-1) == gdn.GDN_ERR_RANGE
    assert call(d, ws=None) == gdn.GDN_ERR_ARG
    assert call(d, ws_bytes=4 * 64 * 32 * 128 - 4) == gdn.GDN_ERR_ARG
    assert call(d, a=[ctypes.c_void_p(0x1004)] + args[1:]) == gdn.GDN_ERR_ARG
    assert call(d, a=args[:3] + [None] + args[4:]) == gdn.GDN_ERR_ARG
    bad = gdn.make_dims(W.CHUNKED_PREFILL)
    bad.d_k = 96
    assert call(bad) == gdn.GDN_ERR_SHAPE


def test_snapshot_restore_validation():
    """gdn_snapshot / gdn_restore reject bad arguments before any launch; n == 0 is a no-op."""
    L = _lib_or_skip()
    d = _dims(n_pool=4)
    bufs = [FAKE] * 4
    for fn in (L.gdn_snapshot, L.gdn_restore):
        assert fn(ctypes.byref(d), *bufs, None, 0, None) == gdn.GDN_OK
        assert fn(ctypes.byref(d), *bufs, FAKE, -1, None) == gdn.GDN_ERR_RANGE
        assert fn(ctypes.byref(d), *bufs, FAKE, 5, None) == gdn.GDN_ERR_RANGE
        assert fn(ctypes.byref(d), *bufs, None, 2, None) == gdn.GDN_ERR_ARG
        assert fn(ctypes.byref(d), None, *bufs[1:], FAKE, 2, None) == gdn.GDN_ERR_ARG
        mis = ctypes.c_void_p(0x1008)
        assert fn(ctypes.byref(d), *bufs[:3], mis, FAKE, 2, None) == gdn.GDN_ERR_ARG
        bad = _dims(n_pool=4, d_conv=3)
        assert fn(ctypes.byref(bad), *bufs, FAKE, 1, None) == gdn.GDN_ERR_SHAPE


def test_rollback_layers_validation():
    """gdn_rollback_layers checks every descriptor, their agreement and buffer ownership before
    any launch; n == 0 is a no-op."""
    L = _lib_or_skip()
    d = _dims(n_pool=4)

    def cap(base, t_cap=16, mode=gdn.GDN_CHAIN, dims=d):
        return gdn.gdn_capture(dims, base, base + 0x100, base + 0x200, base + 0x300, t_cap, mode)

    def arr(*caps):
        return (gdn.gdn_capture * len(caps))(*caps)

    two = arr(cap(0x1000), cap(0x2000))
    assert L.gdn_rollback_layers(two, 2, None, None, 0, None) == gdn.GDN_OK
    assert L.gdn_rollback_layers(None, 2, FAKE, FAKE, 1, None) == gdn.GDN_ERR_ARG
    assert L.gdn_rollback_layers(two, 0, FAKE, FAKE, 1, None) == gdn.GDN_ERR_RANGE
    assert L.gdn_rollback_layers(two, 2, None, None, 2, None) == gdn.GDN_ERR_ARG
    assert L.gdn_rollback_layers(two, 2, FAKE, FAKE, 5, None) == gdn.GDN_ERR_RANGE
    assert L.gdn_rollback_layers(two, 2, FAKE, FAKE, -1, None) == gdn.GDN_ERR_RANGE
    # layers that disagree in t_cap, mode or dims
    assert L.gdn_rollback_layers(arr(cap(0x1000), cap(0x2000, t_cap=8)), 2, FAKE, FAKE, 1, None) == gdn.GDN_ERR_ARG
    assert L.gdn_rollback_layers(arr(cap(0x1000), cap(0x2000, mode=gdn.GDN_TREE)), 2, FAKE, FAKE, 1,
                                 None) == gdn.GDN_ERR_ARG
    assert L.gdn_rollback_layers(arr(cap(0x1000), cap(0x2000, dims=_dims(n_pool=5))), 2, FAKE, FAKE, 1,
                                 None) == gdn.GDN_ERR_ARG
    # two layers restoring into the same state buffer
    assert L.gdn_rollback_layers(arr(cap(0x1000), cap(0x1000)), 2, FAKE, FAKE, 1, None) == gdn.GDN_ERR_ARG
    # a bad descriptor anywhere: its own check's code, naming the layer
    bad = gdn.gdn_capture(d, 0x3000, 0x3100, 0x3200, 0x3308, 16, gdn.GDN_CHAIN)
    assert L.gdn_rollback_layers(arr(cap(0x1000), bad), 2, FAKE, FAKE, 1, None) == gdn.GDN_ERR_ARG
    assert "layer 1" in gdn.last_error()
    bad_shape = cap(0x3000, dims=_dims(n_pool=4, d_conv=3))
    assert L.gdn_rollback_layers(arr(bad_shape), 1, FAKE, FAKE, 1, None) == gdn.GDN_ERR_SHAPE


def test_graph_validation():
    """gdn_graph_create rejects bad arguments before it records anything (no HIP call is made
    for these); launch of a NULL graph fails, destroy of NULL is a no-op."""
    L = _lib_or_skip()
    d = _dims(n_pool=4)
    lay = gdn.gdn_layer(*([0x1000] * 13))
    arr = (gdn.gdn_layer * 2)(lay, lay)
    h = ctypes.c_void_p(None)
    VR = gdn.GDN_GRAPH_VERIFY | gdn.GDN_GRAPH_ROLLBACK

    def create(dims=d, layers=arr, n_layers=2, t_cap=16, n_tok=16, slots=FAKE, n_batch=1, acc=FAKE,
               phases=VR, out=ctypes.byref(h)):
        return L.gdn_graph_create(ctypes.byref(dims) if dims is not None else None, layers, n_layers,
                                  t_cap, n_tok, slots, n_batch, acc, phases, out)

    assert create(out=None) == gdn.GDN_ERR_ARG
    assert create(dims=None) == gdn.GDN_ERR_ARG
    assert create(layers=None) == gdn.GDN_ERR_ARG
    assert create(dims=_dims(n_pool=4, flags=gdn.GDN_F_CHECK_INDICES)) == gdn.GDN_ERR_ARG
    assert "cannot be recorded" in gdn.last_error()
    assert create(phases=0) == gdn.GDN_ERR_ARG
    assert create(phases=0x4) == gdn.GDN_ERR_ARG
    assert create(n_layers=0) == gdn.GDN_ERR_RANGE
    assert create(t_cap=8) == gdn.GDN_ERR_RANGE
    assert create(n_tok=0) == gdn.GDN_ERR_RANGE
    assert create(acc=None) == gdn.GDN_ERR_ARG
    assert create(slots=None) == gdn.GDN_ERR_ARG
    bad = gdn.gdn_layer(*([0x1000] * 12 + [0]))
    assert create(layers=(gdn.gdn_layer * 2)(lay, bad)) == gdn.GDN_ERR_ARG
    assert "layer 1" in gdn.last_error()
    assert h.value is None
    assert L.gdn_graph_launch(None, None) == gdn.GDN_ERR_ARG
    assert L.gdn_graph_destroy(None) == gdn.GDN_OK


def test_linear_validation():
    """gdn_linear checks pointers, shapes and the column segments before any launch."""
    L = _lib_or_skip()

    def segs(*spec):
        return (gdn.gdn_out_seg * len(spec))(*[gdn.gdn_out_seg(n0, n1, ld, dt, sg, 0x2000)
                                                for (n0, n1, ld, dt, sg) in spec])

    good = segs((0, 100, 100, gdn.GDN_BF16, 0), (100, 164, 64, gdn.GDN_F32, 1))

    def call(x=FAKE, w=FAKE, M=8, N=164, K=128, s=good, n=2):
        return L.gdn_linear(x, w, M, N, K, s, n, None)

    assert call(x=None) == gdn.GDN_ERR_ARG
    assert call(w=ctypes.c_void_p(0x1008)) == gdn.GDN_ERR_ARG
    assert call(M=0) == gdn.GDN_ERR_SHAPE
    assert call(K=96) == gdn.GDN_ERR_SHAPE
    assert call(K=0) == gdn.GDN_ERR_SHAPE
    assert call(n=0) == gdn.GDN_ERR_ARG
    assert call(n=5) == gdn.GDN_ERR_ARG
    assert call(N=200) == gdn.GDN_ERR_ARG                      # segments end short of N
    assert call(s=segs((0, 100, 100, 1, 0), (90, 164, 74, 0, 0))) == gdn.GDN_ERR_ARG   # overlap
    assert call(s=segs((0, 100, 99, 1, 0), (100, 164, 64, 0, 0))) == gdn.GDN_ERR_ARG   # ld too small
    assert call(s=segs((0, 100, 100, 7, 0), (100, 164, 64, 0, 0))) == gdn.GDN_ERR_DTYPE
    bad_ptr = (gdn.gdn_out_seg * 1)(gdn.gdn_out_seg(0, 164, 164, 1, 0, None))
    assert call(s=bad_ptr, n=1) == gdn.GDN_ERR_ARG
