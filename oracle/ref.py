"""Python front end of the fp64 C oracle (test infrastructure only).

Every function here either calls the C oracle (gdn_oracle.c) or is a plain copy that the
capture / rollback contract defines:

* chain verify: per-position capture, final state, gated output (lucebox-hub internal.h,
  struct TargetCache, ssm_intermediate / conv_input_cache comments);
* rollback: the state after accepted position a is capture[a]; the conv state is rows
  a+1 .. a+3 of the conv input window (same comments: "commits t = commit_n - 1", slice
  [commit_n .. commit_n + kernel - 2]); accepted_idx = K - trim (hf2q qwen35_target.rs,
  Qwen35DFlashTarget::rollback_kv);
* tree verify: every node evaluated as the chain along its root path (internal.h,
  QwenGraphInputs::parent_ids);
* prefill: the chain over the whole sequence without capture.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgdn_oracle.so")

F_QK_NORM_SILU = 1

_lib = None


class _Dims(ctypes.Structure):
    _fields_ = [("n_kh", ctypes.c_int32), ("n_vh", ctypes.c_int32), ("d_k", ctypes.c_int32),
                ("d_v", ctypes.c_int32), ("d_conv", ctypes.c_int32), ("flags", ctypes.c_int32),
                ("eps", ctypes.c_double)]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH) or (
                os.path.getmtime(LIB_PATH) < os.path.getmtime(os.path.join(HERE, "gdn_oracle.c"))):
            from oracle.build import build
            build()
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        i = ctypes.c_int
        L.ora_verify.argtypes = [ctypes.POINTER(_Dims), i, i, i] + [P] * 11 + [i, P, P, P, P, P, P, i]
        L.ora_verify.restype = i
        L.ora_tree.argtypes = [ctypes.POINTER(_Dims), i, i, i] + [P] * 12 + [i, P, P, P, P, i]
        L.ora_tree.restype = i
        L.ora_tree_conv.argtypes = [ctypes.POINTER(_Dims), i, i, i, P, P, P, P, P]
        L.ora_tree_conv.restype = i
        L.ora_conv.argtypes = [ctypes.POINTER(_Dims), i, P, P, P, P]
        L.ora_conv.restype = None
        L.ora_gate.argtypes = [ctypes.c_double] * 3
        L.ora_gate.restype = ctypes.c_double
        L.ora_softplus.argtypes = [ctypes.c_double]
        L.ora_softplus.restype = ctypes.c_double
        L.ora_norm_gate.argtypes = [i, P, P, P, ctypes.c_double, P]
        L.ora_norm_gate.restype = None
        L.ora_max_threads.argtypes = []
        L.ora_max_threads.restype = i
        _lib = L
    return _lib


def _dims(shape, flags: int = 0, eps: float = 1e-6) -> _Dims:
    return _Dims(shape.n_kh, shape.n_vh, shape.d_k, shape.d_v, shape.d_conv, flags, eps)


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def _i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def all_units(shape) -> tuple:
    b, h = np.meshgrid(np.arange(shape.n_batch), np.arange(shape.n_vh), indexing="ij")
    return _i32(b.ravel()), _i32(h.ravel())


def verify_units(shape, inp: dict, units: Optional[tuple] = None, *, n_tok: Optional[int] = None,
                 capture: bool = True, want_o: bool = False, flags: int = 0, eps: float = 1e-6,
                 n_threads: int = 0) -> dict:
    """Chain verify of the listed (batch entry, value head) units.

    Returns fp64 arrays: state [U][d_v][d_k], cap [U][T][d_v][d_k] (if capture),
    y [U][T][d_v], o [U][T][d_v] (if want_o), plus the unit lists.
    ``n_tok`` (<= the generated T) verifies only the first n_tok tokens of each entry.
    """
    T_all = shape.n_tok
    T = T_all if n_tok is None else int(n_tok)
    ub, uh = all_units(shape) if units is None else (_i32(units[0]), _i32(units[1]))
    U = len(ub)
    dv, dk = shape.d_v, shape.d_k
    qkv = _f32(inp["qkv"][:, :T])
    z = _f32(inp["z"][:, :T])
    alpha = _f32(inp["alpha"][:, :T])
    beta = _f32(inp["beta"][:, :T])
    st = np.empty((U, dv, dk))
    cap = np.empty((U, T, dv, dk)) if capture else None
    y = np.empty((U, T, dv))
    o = np.empty((U, T, dv)) if want_o else None
    rc = lib().ora_verify(ctypes.byref(_dims(shape, flags, eps)), T, shape.n_batch, shape.n_pool,
                          _ptr(qkv), _ptr(z), _ptr(alpha), _ptr(beta), _ptr(_f32(inp["A_log"])),
                          _ptr(_f32(inp["dt_bias"])), _ptr(_f32(inp["conv_w"])),
                          _ptr(_f32(inp["norm_w"])), _ptr(_f32(inp["state"])),
                          _ptr(_f32(inp["conv_state"])), _ptr(_i32(inp["slot_ids"])), U,
                          _ptr(ub), _ptr(uh), _ptr(st), _ptr(cap), _ptr(y), _ptr(o), n_threads)
    if rc != 0:
        raise ValueError("oracle: index out of range")
    out = {"state": st, "y": y, "units": (ub, uh)}
    if capture:
        out["cap"] = cap
    if want_o:
        out["o"] = o
    return out


def conv_window(shape, inp: dict, n_tok: Optional[int] = None) -> np.ndarray:
    """The conv input window concat(conv_state[slot], qkv rows), [B][3+T][C] fp32 (a copy)."""
    T = shape.n_tok if n_tok is None else int(n_tok)
    cs = inp["conv_state"][inp["slot_ids"]]
    return np.concatenate([cs, inp["qkv"][:, :T]], axis=1).astype(np.float32)


def conv(shape, inp: dict, b: int, n_tok: Optional[int] = None) -> np.ndarray:
    """Post-conv activations of batch entry b, [T][C] fp64."""
    T = shape.n_tok if n_tok is None else int(n_tok)
    C = shape.conv_channels
    out = np.empty((T, C))
    s = int(inp["slot_ids"][b])
    lib().ora_conv(ctypes.byref(_dims(shape)), T, _ptr(_f32(inp["qkv"][b, :T])),
                   _ptr(_f32(inp["conv_state"][s])), _ptr(_f32(inp["conv_w"])), _ptr(out))
    return out


def gate(A_log: float, dt_bias: float, alpha: float) -> float:
    return lib().ora_gate(float(A_log), float(dt_bias), float(alpha))


def softplus(x: float) -> float:
    return lib().ora_softplus(float(x))


def norm_gate(o: np.ndarray, z: np.ndarray, w: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    o = np.ascontiguousarray(o, dtype=np.float64)
    y = np.empty_like(o)
    lib().ora_norm_gate(len(o), _ptr(o), _ptr(_f32(z)), _ptr(_f32(w)), eps, _ptr(y))
    return y


def verify_pool(shape, inp: dict, *, n_tok: Optional[int] = None, flags: int = 0,
                eps: float = 1e-6, n_threads: int = 0) -> dict:
    """Chain verify of a whole (small) call, pool-level results (fp64 except conv copies):

    state [P][H_v][d_v][d_k] (untouched slots keep the input), conv_state [P][3][C] fp32,
    cap_ssm [P][T][H_v][d_v][d_k] (NaN where nothing was written), cap_conv [P][3+T][C] fp32,
    out [B][T][H_v][d_v].
    """
    T = shape.n_tok if n_tok is None else int(n_tok)
    P, B, Hv, dv, dk = shape.n_pool, shape.n_batch, shape.n_vh, shape.d_v, shape.d_k
    r = verify_units(shape, inp, n_tok=T, flags=flags, eps=eps, n_threads=n_threads)
    ub, uh = r["units"]
    state = inp["state"].astype(np.float64).copy()
    cap = np.full((P, T, Hv, dv, dk), np.nan)
    out = np.empty((B, T, Hv, dv))
    for u in range(len(ub)):
        b, h = int(ub[u]), int(uh[u])
        s = int(inp["slot_ids"][b])
        state[s, h] = r["state"][u]
        cap[s, :, h] = r["cap"][u]
        out[b, :, h] = r["y"][u]
    win = conv_window(shape, inp, T)
    conv_state = inp["conv_state"].copy()
    cap_conv = np.full((P, 3 + T, shape.conv_channels), np.nan, dtype=np.float32)
    for b in range(B):
        s = int(inp["slot_ids"][b])
        conv_state[s] = win[b, T:T + 3]
        cap_conv[s] = win[b]
    return {"state": state, "conv_state": conv_state, "cap_ssm": cap, "cap_conv": cap_conv,
            "out": out}


def rollback_chain(state: np.ndarray, conv_state: np.ndarray, cap_ssm: np.ndarray,
                   cap_conv: np.ndarray, slot: int, a: int) -> None:
    """In place: state[slot] <- cap_ssm[slot][a]; conv_state[slot] <- cap_conv[slot][a+1 .. a+3]."""
    state[slot] = cap_ssm[slot, a]
    conv_state[slot] = cap_conv[slot, a + 1:a + 4]


def rollback_tree(state: np.ndarray, conv_state: np.ndarray, cap_ssm: np.ndarray,
                  cap_conv_tree: np.ndarray, slot: int, a: int) -> None:
    """In place: state[slot] <- cap_ssm[slot][a]; conv_state[slot] <- cap_conv_tree[slot][a]."""
    state[slot] = cap_ssm[slot, a]
    conv_state[slot] = cap_conv_tree[slot, a]


def accepted_index(n_tokens_max: int, trim: int) -> Optional[int]:
    """accepted_idx = n_tokens_max - 1 - trim; None when trim == 0 (nothing to undo) or when
    trim >= n_tokens_max (more than was verified).  hf2q qwen35_target.rs, rollback_kv."""
    if trim == 0 or trim >= n_tokens_max:
        return None
    return n_tokens_max - 1 - trim


def tree_units(shape, inp: dict, units: Optional[tuple] = None, *, flags: int = 0,
               eps: float = 1e-6, n_threads: int = 0) -> dict:
    """Tree verify of the listed units: cap [U][T][d_v][d_k] and y [U][T][d_v] (fp64)."""
    ub, uh = all_units(shape) if units is None else (_i32(units[0]), _i32(units[1]))
    U, T = len(ub), shape.n_tok
    cap = np.empty((U, T, shape.d_v, shape.d_k))
    y = np.empty((U, T, shape.d_v))
    rc = lib().ora_tree(ctypes.byref(_dims(shape, flags, eps)), T, shape.n_batch, shape.n_pool,
                        _ptr(_f32(inp["qkv"])), _ptr(_f32(inp["z"])), _ptr(_f32(inp["alpha"])),
                        _ptr(_f32(inp["beta"])), _ptr(_f32(inp["A_log"])),
                        _ptr(_f32(inp["dt_bias"])), _ptr(_f32(inp["conv_w"])),
                        _ptr(_f32(inp["norm_w"])), _ptr(_f32(inp["state"])),
                        _ptr(_f32(inp["conv_state"])), _ptr(_i32(inp["slot_ids"])),
                        _ptr(_i32(inp["parent"])), U, _ptr(ub), _ptr(uh), _ptr(cap), _ptr(y),
                        n_threads)
    if rc != 0:
        raise ValueError("oracle: malformed parent array or index")
    return {"cap": cap, "y": y, "units": (ub, uh)}


def tree_conv(shape, inp: dict) -> np.ndarray:
    """Per-node conv state of a tree call, [B][T][3][C] fp32 (a copy of inputs)."""
    T, B, C = shape.n_tok, shape.n_batch, shape.conv_channels
    cap = np.empty((B, T, 3, C), dtype=np.float32)
    rc = lib().ora_tree_conv(ctypes.byref(_dims(shape)), T, B, shape.n_pool,
                             _ptr(_f32(inp["qkv"])), _ptr(_f32(inp["conv_state"])),
                             _ptr(_i32(inp["slot_ids"])), _ptr(_i32(inp["parent"])), _ptr(cap))
    if rc != 0:
        raise ValueError("oracle: malformed parent array or index")
    return cap


def prefill_units(shape, inp: dict, units: Optional[tuple] = None, *, flags: int = 0,
                  eps: float = 1e-6, n_threads: int = 0) -> dict:
    """Prefill = the chain over the whole sequence without capture (state and y per unit)."""
    return verify_units(shape, inp, units, capture=False, flags=flags, eps=eps,
                        n_threads=n_threads)


def max_threads() -> int:
    return lib().ora_max_threads()


def sample_units(shape, n: int, seed: int = 1234) -> tuple:
    """n distinct (batch entry, value head) units drawn at random (always including the
    first and last unit)."""
    rng = np.random.default_rng(seed)
    total = shape.n_batch * shape.n_vh
    n = min(n, total)
    pick = set([0, total - 1])
    pick.update(int(x) for x in rng.choice(total, size=max(0, n - 2), replace=False))
    pick = sorted(pick)[:max(n, 2)] if total >= 2 else [0]
    idx = np.array(pick)
    return _i32(idx // shape.n_vh), _i32(idx % shape.n_vh)


__all__: Sequence[str] = [
    "verify_units", "verify_pool", "conv_window", "conv", "gate", "softplus", "norm_gate",
    "rollback_chain", "rollback_tree", "accepted_index", "tree_units", "tree_conv",
    "prefill_units", "max_threads", "sample_units", "all_units", "F_QK_NORM_SILU",
]
