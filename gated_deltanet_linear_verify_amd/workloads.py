"""Seeded synthetic inputs for the Gated DeltaNet verify / rollback / tree / prefill path.

This module only draws random numbers and rounds them to the storage dtype. It holds none of
the method's arithmetic (no conv, gate, recurrence or norm), so both the CPU oracle and the HIP
path consume exactly the same values without sharing any computation.

Recipe (fixed draw order, numpy PCG64 ``default_rng(seed)``, fp64 draws, then fp32, then the
activation dtype with round-to-nearest-even through torch):

  1. qkv    ~ N(0, 1), shape [B][T][C]; every q and k head slice (d_k channels) is divided by
              its Euclidean length, v is left as drawn.
  2. z      ~ N(0, 1), shape [B][T][H_v][d_v]
  3. alpha  ~ N(0, 1), shape [B][T][H_v]
  4. beta   = sigmoid(N(0, 1)), shape [B][T][H_v]
  5. A_log  ~ U(lo, hi) with (lo, hi) = (0, 1), or (-8, -4) for the weak-decay variant, [H_v]
  6. dt_bias ~ N(0, 0.1), [H_v]
  7. state  ~ N(0, 0.1), [P][H_v][d_v][d_k]   (zero when ``zero_state``)
  8. conv_state: three past input rows drawn like qkv (step 1), [P][3][C], kept in fp32
  9. conv_w ~ N(0, 0.5), [C][4]
 10. norm_w = 1 + N(0, 0.1), [d_v]
 11. slot_ids = permutation(P)[:B]
 12. trims ~ U{0 .. T-1}, [B]
 13. (tree workloads) parent arrays and accepted nodes, see ``random_tree``.

Channel order of the fused qkv stream: q block [H_k][d_k], then k block [H_k][d_k], then
v block [H_v][d_v].  N(mu, sigma) means standard deviation sigma.
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

F32 = 0
BF16 = 1
DTYPE_NAMES = {F32: "f32", BF16: "bf16"}


@dataclasses.dataclass(frozen=True)
class Shape:
    """Problem geometry of one call."""

    n_kh: int
    n_vh: int
    d_k: int
    d_v: int
    n_pool: int          # P: slots in the state pool
    n_batch: int         # B: batch entries per call
    n_tok: int           # T: tokens (chain), nodes (tree) or sequence length (prefill)
    act_dtype: int = BF16
    out_dtype: int = BF16
    d_conv: int = 4

    @property
    def conv_channels(self) -> int:
        return 2 * self.n_kh * self.d_k + self.n_vh * self.d_v


# The five workloads of the verify path, named after what they are.
TINY_VERIFY = Shape(n_kh=4, n_vh=4, d_k=64, d_v=64, n_pool=1, n_batch=1, n_tok=4,
                    act_dtype=F32, out_dtype=F32)
SINGLE_SLOT_VERIFY = Shape(n_kh=16, n_vh=32, d_k=128, d_v=128, n_pool=1, n_batch=1, n_tok=16)
MULTI_SLOT_VERIFY = Shape(n_kh=16, n_vh=32, d_k=128, d_v=128, n_pool=64, n_batch=64, n_tok=16)
TREE_VERIFY = Shape(n_kh=16, n_vh=32, d_k=128, d_v=128, n_pool=8, n_batch=8, n_tok=64)
CHUNKED_PREFILL = Shape(n_kh=16, n_vh=32, d_k=128, d_v=128, n_pool=1, n_batch=1, n_tok=8192)

WORKLOADS = {
    "tiny_verify": TINY_VERIFY,
    "single_slot_verify": SINGLE_SLOT_VERIFY,
    "multi_slot_verify": MULTI_SLOT_VERIFY,
    "tree_verify": TREE_VERIFY,
    "chunked_prefill": CHUNKED_PREFILL,
}

TREE_MAX_DEPTH = 8


def round_to(x: np.ndarray, dtype: int) -> np.ndarray:
    """fp64 -> fp32 -> (optionally) bf16, returned as fp32 holding the rounded values."""
    x32 = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == F32:
        return x32
    import torch  # round-to-nearest-even bf16 conversion

    return torch.from_numpy(x32).to(torch.bfloat16).to(torch.float32).numpy()


def _unit_rows(rng: np.random.Generator, lead: tuple, shape: Shape) -> np.ndarray:
    """Rows of the fused qkv stream with q and k head slices of unit length (step 1)."""
    C = shape.conv_channels
    x = rng.standard_normal(lead + (C,))
    nqk = shape.n_kh * shape.d_k
    for blk in range(2):
        sl = x[..., blk * nqk:(blk + 1) * nqk]
        heads = sl.reshape(lead + (shape.n_kh, shape.d_k))
        heads /= np.linalg.norm(heads, axis=-1, keepdims=True)
        x[..., blk * nqk:(blk + 1) * nqk] = heads.reshape(lead + (nqk,))
    return x


def make_inputs(shape: Shape, seed: int = 0, *, weak_decay: bool = False,
                zero_state: bool = False) -> dict:
    """All inputs of one call as fp32 numpy arrays holding dtype-rounded values.

    Keys: qkv, z, alpha, beta, A_log, dt_bias, state, conv_state, conv_w, norm_w,
    slot_ids (int32), trims (int32).
    """
    rng = np.random.default_rng(seed)
    B, T, P = shape.n_batch, shape.n_tok, shape.n_pool
    Hv, dv, dk = shape.n_vh, shape.d_v, shape.d_k
    act = shape.act_dtype
    qkv = _unit_rows(rng, (B, T), shape)
    z = rng.standard_normal((B, T, Hv, dv))
    alpha = rng.standard_normal((B, T, Hv))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, Hv))))
    lo, hi = (-8.0, -4.0) if weak_decay else (0.0, 1.0)
    A_log = rng.uniform(lo, hi, Hv)
    dt_bias = rng.normal(0.0, 0.1, Hv)
    state = rng.normal(0.0, 0.1, (P, Hv, dv, dk))
    if zero_state:
        state = np.zeros_like(state)
    conv_state = _unit_rows(rng, (P, shape.d_conv - 1), shape)
    conv_w = rng.normal(0.0, 0.5, (shape.conv_channels, shape.d_conv))
    norm_w = 1.0 + rng.normal(0.0, 0.1, dv)
    slot_ids = rng.permutation(P)[:B].astype(np.int32)
    trims = rng.integers(0, T, size=B).astype(np.int32)
    return {
        "qkv": round_to(qkv, act),
        "z": round_to(z, act),
        "alpha": round_to(alpha, act),
        "beta": round_to(beta, act),
        "A_log": round_to(A_log, F32),
        "dt_bias": round_to(dt_bias, F32),
        "state": round_to(state, F32),
        "conv_state": round_to(conv_state, F32),
        "conv_w": round_to(conv_w, F32),
        "norm_w": round_to(norm_w, F32),
        "slot_ids": slot_ids,
        "trims": trims,
    }


def random_tree(rng: np.random.Generator, n_nodes: int,
                max_depth: int = TREE_MAX_DEPTH) -> np.ndarray:
    """Parent array of a random draft tree: node 0 is the root (parent -1); node i > 0 takes a
    parent uniformly among earlier nodes whose depth is below ``max_depth``."""
    parent = np.full(n_nodes, -1, dtype=np.int32)
    depth = np.zeros(n_nodes, dtype=np.int64)
    for i in range(1, n_nodes):
        cand = np.nonzero(depth[:i] < max_depth)[0]
        p = int(cand[rng.integers(0, len(cand))])
        parent[i] = p
        depth[i] = depth[p] + 1
    return parent


def tree_accept(rng: np.random.Generator, parent: np.ndarray) -> int:
    """A random accepted node: the end of a random prefix of the root path of a random leaf."""
    n = len(parent)
    has_child = np.zeros(n, dtype=bool)
    has_child[parent[parent >= 0]] = True
    leaves = np.nonzero(~has_child)[0]
    leaf = int(leaves[rng.integers(0, len(leaves))])
    path = [leaf]
    while parent[path[-1]] >= 0:
        path.append(int(parent[path[-1]]))
    path.reverse()
    return int(path[rng.integers(0, len(path))])


def make_tree_inputs(shape: Shape, seed: int = 0, **kw) -> dict:
    """Chain inputs plus per-batch-entry parent arrays [B][T] and accepted nodes [B]."""
    inp = make_inputs(shape, seed, **kw)
    rng = np.random.default_rng([seed, 1])
    parents = np.stack([random_tree(rng, shape.n_tok) for _ in range(shape.n_batch)])
    accepted = np.array([tree_accept(rng, p) for p in parents], dtype=np.int32)
    inp["parent"] = parents.astype(np.int32)
    inp["accepted"] = accepted
    return inp


def tree_depths(parent: np.ndarray) -> np.ndarray:
    """Depth of every node (root 0); parent[i] < i is assumed."""
    d = np.zeros(len(parent), dtype=np.int64)
    for i, p in enumerate(parent):
        d[i] = 0 if p < 0 else d[p] + 1
    return d


def chain_parents(n: int) -> np.ndarray:
    """The parent array of a linear chain (node i hangs off node i-1)."""
    return (np.arange(n, dtype=np.int32) - 1).astype(np.int32)


def shape_with(shape: Shape, **kw) -> Shape:
    return dataclasses.replace(shape, **kw)


def describe(shape: Shape) -> dict:
    return {
        "n_kh": shape.n_kh, "n_vh": shape.n_vh, "d_k": shape.d_k, "d_v": shape.d_v,
        "n_pool": shape.n_pool, "n_batch": shape.n_batch, "n_tok": shape.n_tok,
        "act": DTYPE_NAMES[shape.act_dtype], "out": DTYPE_NAMES[shape.out_dtype],
    }


def digest(inputs: dict, extra: Optional[dict] = None) -> str:
    """A stable hash of every generated array (determinism check)."""
    import hashlib

    h = hashlib.sha256()
    for k in sorted(inputs):
        a = np.ascontiguousarray(inputs[k])
        h.update(k.encode())
        h.update(str(a.dtype).encode())
        h.update(str(a.shape).encode())
        h.update(a.tobytes())
    if extra:
        h.update(repr(sorted(extra.items())).encode())
    return h.hexdigest()


# Width of the pages' model (TargetWeights n_embd), the input of the GDN block's projections.
HIDDEN = 5120


def make_block_inputs(shape: Shape, hidden: int, seed: int = 0) -> dict:
    """Inputs of one GDN block call: make_inputs' layer inputs (state, conv state, gate and norm
    parameters, conv taps, slots; its qkv / z / alpha / beta are replaced by the block's own
    projections) plus x [B][T][hidden] ~ N(0, 1) and random projection weights, one output
    feature per row with the input index fastest: w_qkv [C][hidden], w_z [H_v d_v][hidden],
    w_beta and w_alpha [H_v][hidden], each ~ N(0, 1/hidden), and w_out [hidden][H_v d_v] ~
    N(0, 1/(H_v d_v)).  All bf16-rounded (fp32 arrays holding bf16 values)."""
    inp = make_inputs(shape, seed)
    for k in ("qkv", "z", "alpha", "beta"):
        del inp[k]
    rng = np.random.default_rng(seed + 7919)
    B, T, Hv, dv, C = shape.n_batch, shape.n_tok, shape.n_vh, shape.d_v, shape.conv_channels
    s_in, s_out = 1.0 / np.sqrt(hidden), 1.0 / np.sqrt(Hv * dv)
    inp["x"] = round_to(rng.standard_normal((B, T, hidden)), BF16)
    inp["w_qkv"] = round_to(rng.normal(0.0, s_in, (C, hidden)), BF16)
    inp["w_z"] = round_to(rng.normal(0.0, s_in, (Hv * dv, hidden)), BF16)
    inp["w_beta"] = round_to(rng.normal(0.0, s_in, (Hv, hidden)), BF16)
    inp["w_alpha"] = round_to(rng.normal(0.0, s_in, (Hv, hidden)), BF16)
    inp["w_out"] = round_to(rng.normal(0.0, s_out, (hidden, Hv * dv)), BF16)
    return inp
