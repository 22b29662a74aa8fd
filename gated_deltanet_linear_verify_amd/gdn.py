"""ctypes binding of libgdn.so (include/gdn.h), with the same names as the C entry points.

Argument marshalling only: tensors are passed as device pointers, the current torch stream as
the HIP stream, and every non-zero status becomes a ``GdnError``.  There is no fallback: if the
library is missing, loading fails loudly.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libgdn.so")

GDN_OK, GDN_ERR_ARG, GDN_ERR_SHAPE, GDN_ERR_DTYPE, GDN_ERR_RANGE, GDN_ERR_HIP = range(6)
GDN_F32, GDN_BF16 = 0, 1
GDN_CHAIN, GDN_TREE = 0, 1
GDN_F_QK_NORM_SILU = 0x1
GDN_F_CHECK_INDICES = 0x2
GDN_F_DEFER_COMMIT = 0x4

EXPORTS = ("gdn_verify", "gdn_verify_resume", "gdn_verify_tree", "gdn_rollback", "gdn_rollback_batch", "gdn_rollback_trim",
           "gdn_prefill", "gdn_prefill_noalloc", "gdn_prefill_workspace_bytes", "gdn_capture_bytes", "gdn_reset",
           "gdn_snapshot", "gdn_restore", "gdn_rollback_layers", "gdn_graph_create", "gdn_graph_launch",
           "gdn_graph_destroy", "gdn_linear", "gdn_last_error", "gdn_version")


class GdnError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"[gdn status {code}] {msg}")
        self.code = code


class gdn_dims(ctypes.Structure):
    _fields_ = [("n_kh", ctypes.c_int32), ("n_vh", ctypes.c_int32), ("d_k", ctypes.c_int32),
                ("d_v", ctypes.c_int32), ("d_conv", ctypes.c_int32), ("n_pool", ctypes.c_int32),
                ("act_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
                ("flags", ctypes.c_uint32), ("eps", ctypes.c_float)]


class gdn_capture(ctypes.Structure):
    _fields_ = [("dims", gdn_dims), ("ssm", ctypes.c_void_p), ("conv", ctypes.c_void_p),
                ("state", ctypes.c_void_p), ("conv_state", ctypes.c_void_p),
                ("t_cap", ctypes.c_int32), ("mode", ctypes.c_int32)]


class gdn_layer(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("state", "conv_state", "qkv", "z", "alpha", "beta", "A_log",
                                                "dt_bias", "conv_w", "norm_w", "cap_ssm", "cap_conv", "out")]


class gdn_out_seg(ctypes.Structure):
    _fields_ = [("n0", ctypes.c_int32), ("n1", ctypes.c_int32), ("ld", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("sigmoid", ctypes.c_int32), ("ptr", ctypes.c_void_p)]


GDN_GRAPH_VERIFY = 0x1
GDN_GRAPH_ROLLBACK = 0x2

_lib = None


def lib() -> ctypes.CDLL:
    """Load libgdn.so (built in-tree by ``gated_deltanet_linear_verify_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m gated_deltanet_linear_verify_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, I, S = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        D = ctypes.POINTER(gdn_dims)
        Cp = ctypes.POINTER(gdn_capture)
        L.gdn_verify.argtypes = [D, P, P, P, P, P, P, P, P, P, P, Cp, P, I, P, I, P]
        L.gdn_verify_tree.argtypes = [D, P, P, P, P, P, P, P, P, P, P, P, Cp, P, I, P, I, P]
        L.gdn_verify_resume.argtypes = [D, P, P, P, P, P, P, P, P, P, P, Cp, P, I, P, P, I, P]
        L.gdn_rollback.argtypes = [Cp, I, I, P]
        L.gdn_rollback_batch.argtypes = [Cp, P, P, I, P]
        L.gdn_rollback_trim.argtypes = [Cp, I, I, I, P]
        L.gdn_prefill.argtypes = [D, P, P, P, P, P, P, P, P, P, P, P, I, I, P, S, P]
        L.gdn_prefill_noalloc.argtypes = [D, P, P, P, P, P, P, P, P, P, P, P, I, I, P]
        L.gdn_prefill_workspace_bytes.argtypes = [D, I]
        L.gdn_prefill_workspace_bytes.restype = S
        L.gdn_capture_bytes.argtypes = [D, I, I, ctypes.POINTER(S)]
        L.gdn_capture_bytes.restype = S
        L.gdn_reset.argtypes = [D, P, P, I, P]
        L.gdn_snapshot.argtypes = [D, P, P, P, P, P, I, P]
        L.gdn_restore.argtypes = [D, P, P, P, P, P, I, P]
        L.gdn_rollback_layers.argtypes = [Cp, I, P, P, I, P]
        L.gdn_graph_create.argtypes = [D, ctypes.POINTER(gdn_layer), I, I, I, P, I, P, ctypes.c_uint32,
                                       ctypes.POINTER(ctypes.c_void_p)]
        L.gdn_graph_launch.argtypes = [P, P]
        L.gdn_linear.argtypes = [P, P, I, I, I, ctypes.POINTER(gdn_out_seg), I, P]
        L.gdn_graph_destroy.argtypes = [P]
        for f in ("gdn_verify", "gdn_verify_resume", "gdn_verify_tree", "gdn_rollback", "gdn_rollback_batch",
                  "gdn_rollback_trim", "gdn_prefill", "gdn_prefill_noalloc", "gdn_reset", "gdn_snapshot", "gdn_restore",
                  "gdn_rollback_layers", "gdn_graph_create", "gdn_graph_launch", "gdn_graph_destroy",
                  "gdn_linear"):
            getattr(L, f).restype = ctypes.c_int
        L.gdn_last_error.restype = ctypes.c_char_p
        L.gdn_version.restype = ctypes.c_char_p
        _lib = L
    return _lib


def last_error() -> str:
    return lib().gdn_last_error().decode()


def version() -> str:
    return lib().gdn_version().decode()


def _check(rc: int) -> None:
    if rc != GDN_OK:
        raise GdnError(rc, last_error())


def make_dims(shape, *, flags: int = 0, eps: float = 1e-6, n_pool: Optional[int] = None) -> gdn_dims:
    """gdn_dims from a workloads.Shape."""
    return gdn_dims(shape.n_kh, shape.n_vh, shape.d_k, shape.d_v, shape.d_conv,
                    shape.n_pool if n_pool is None else n_pool, shape.act_dtype, shape.out_dtype,
                    flags, eps)


def _p(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


class Capture:
    """Per-position capture buffers (torch tensors) plus the restore targets."""

    def __init__(self, dims: gdn_dims, ssm, conv, state, conv_state, t_cap: int, mode: int):
        self.dims, self.ssm, self.conv = dims, ssm, conv
        self.state, self.conv_state = state, conv_state
        self.t_cap, self.mode = t_cap, mode
        self.c = gdn_capture(dims, _p(ssm), _p(conv), _p(state), _p(conv_state), t_cap, mode)

    @property
    def ref(self):
        return ctypes.byref(self.c)


def capture_bytes(dims: gdn_dims, t_cap: int, mode: int) -> tuple:
    cb = ctypes.c_size_t(0)
    sb = lib().gdn_capture_bytes(ctypes.byref(dims), t_cap, mode, ctypes.byref(cb))
    return sb, cb.value


def gdn_verify(dims, state, conv_state, qkv, z, alpha, beta, A_log, dt_bias, conv_w, norm_w,
               capture: Optional[Capture], out, n_tok: int, slot_ids, n_batch: int,
               stream=None) -> None:
    _check(lib().gdn_verify(ctypes.byref(dims), _p(state), _p(conv_state), _p(qkv), _p(z),
                            _p(alpha), _p(beta), _p(A_log), _p(dt_bias), _p(conv_w), _p(norm_w),
                            capture.ref if capture is not None else None, _p(out), n_tok,
                            _p(slot_ids), n_batch, _stream(stream)))


def gdn_verify_resume(dims, state, conv_state, qkv, z, alpha, beta, A_log, dt_bias, conv_w, norm_w,
                      capture: Capture, out, n_tok: int, slot_ids, resume_idx, n_batch: int,
                      stream=None) -> None:
    _check(lib().gdn_verify_resume(ctypes.byref(dims), _p(state), _p(conv_state), _p(qkv), _p(z),
                                   _p(alpha), _p(beta), _p(A_log), _p(dt_bias), _p(conv_w),
                                   _p(norm_w), capture.ref if capture is not None else None,
                                   _p(out), n_tok, _p(slot_ids), _p(resume_idx), n_batch,
                                   _stream(stream)))


def gdn_verify_tree(dims, state, conv_state, qkv, z, alpha, beta, A_log, dt_bias, conv_w, norm_w,
                    parent, capture: Capture, out, n_tok: int, slot_ids, n_batch: int,
                    stream=None) -> None:
    _check(lib().gdn_verify_tree(ctypes.byref(dims), _p(state), _p(conv_state), _p(qkv), _p(z),
                                 _p(alpha), _p(beta), _p(A_log), _p(dt_bias), _p(conv_w),
                                 _p(norm_w), _p(parent), capture.ref, _p(out), n_tok,
                                 _p(slot_ids), n_batch, _stream(stream)))


def gdn_rollback(capture: Capture, slot: int, accepted_idx: int, stream=None) -> None:
    _check(lib().gdn_rollback(capture.ref, slot, accepted_idx, _stream(stream)))


def gdn_rollback_batch(capture: Capture, slots, accepted_idx, n: int, stream=None) -> None:
    _check(lib().gdn_rollback_batch(capture.ref, _p(slots), _p(accepted_idx), n, _stream(stream)))


def gdn_rollback_layers(layers, slots, accepted_idx, n: int, stream=None) -> None:
    """One launch (per 64 layers) restoring every layer's capture for the listed slots."""
    arr = (gdn_capture * len(layers))(*[c.c for c in layers])
    _check(lib().gdn_rollback_layers(arr, len(layers), _p(slots), _p(accepted_idx), n, _stream(stream)))


def gdn_linear(x, w, M: int, N: int, K: int, segs, stream=None) -> None:
    """y = x W^T into column segments: segs is a list of (n0, n1, tensor, ld, sigmoid) with the
    tensor's dtype (bf16 or fp32) as the storage type."""
    import torch
    arr = (gdn_out_seg * len(segs))(*[
        gdn_out_seg(n0, n1, ld, GDN_BF16 if t.dtype == torch.bfloat16 else GDN_F32, int(bool(sg)), _p(t))
        for (n0, n1, t, ld, sg) in segs])
    _check(lib().gdn_linear(_p(x), _p(w), M, N, K, arr, len(segs), _stream(stream)))


class Graph:
    """A recorded spec-decode step (gdn_graph_create) over layers given as dicts of torch tensors
    with the gdn_layer field names; replay with launch(), freed by close() or on collection."""

    def __init__(self, dims, layers, t_cap: int, n_tok: int, slot_ids, n_batch: int, accepted_idx,
                 phases: int = GDN_GRAPH_VERIFY | GDN_GRAPH_ROLLBACK):
        arr = (gdn_layer * len(layers))(*[gdn_layer(*[_p(L[n]) for n, _ in gdn_layer._fields_])
                                          for L in layers])
        self._h = ctypes.c_void_p(None)
        self._keep = (layers, slot_ids, accepted_idx)  # the graph holds raw pointers into these
        _check(lib().gdn_graph_create(ctypes.byref(dims), arr, len(layers), t_cap, n_tok, _p(slot_ids),
                                      n_batch, _p(accepted_idx), phases, ctypes.byref(self._h)))

    def launch(self, stream=None) -> None:
        _check(lib().gdn_graph_launch(self._h, _stream(stream)))

    def close(self) -> None:
        if self._h:
            _check(lib().gdn_graph_destroy(self._h))
            self._h = ctypes.c_void_p(None)

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def gdn_rollback_trim(capture: Capture, slot: int, trim: int, n_tok: int, stream=None) -> None:
    _check(lib().gdn_rollback_trim(capture.ref, slot, trim, n_tok, _stream(stream)))


def gdn_prefill_workspace_bytes(dims, n_tok: int) -> int:
    return lib().gdn_prefill_workspace_bytes(ctypes.byref(dims), n_tok)


def gdn_prefill(dims, state, conv_state, qkv, z, alpha, beta, A_log, dt_bias, conv_w, norm_w, out,
                n_tok: int, slot: int, workspace, ws_bytes: int, stream=None) -> None:
    _check(lib().gdn_prefill(ctypes.byref(dims), _p(state), _p(conv_state), _p(qkv), _p(z),
                             _p(alpha), _p(beta), _p(A_log), _p(dt_bias), _p(conv_w), _p(norm_w),
                             _p(out), n_tok, slot, _p(workspace), ws_bytes, _stream(stream)))


def gdn_prefill_noalloc(dims, state, conv_state, qkv, z, alpha, beta, A_log, dt_bias, conv_w, norm_w,
                        out, n_tok: int, slot: int, stream=None) -> None:
    _check(lib().gdn_prefill_noalloc(ctypes.byref(dims), _p(state), _p(conv_state), _p(qkv), _p(z),
                                     _p(alpha), _p(beta), _p(A_log), _p(dt_bias), _p(conv_w),
                                     _p(norm_w), _p(out), n_tok, slot, _stream(stream)))


def gdn_reset(dims, state, conv_state, slot: int, stream=None) -> None:
    _check(lib().gdn_reset(ctypes.byref(dims), _p(state), _p(conv_state), slot, _stream(stream)))


def gdn_snapshot(dims, state, conv_state, snap_state, snap_conv, slots, n: int, stream=None) -> None:
    _check(lib().gdn_snapshot(ctypes.byref(dims), _p(state), _p(conv_state), _p(snap_state), _p(snap_conv),
                              _p(slots), n, _stream(stream)))


def gdn_restore(dims, state, conv_state, snap_state, snap_conv, slots, n: int, stream=None) -> None:
    _check(lib().gdn_restore(ctypes.byref(dims), _p(state), _p(conv_state), _p(snap_state), _p(snap_conv),
                             _p(slots), n, _stream(stream)))
