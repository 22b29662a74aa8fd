"""The projections around the Gated DeltaNet layer and the block they form (test infrastructure
only; fp64).

lucebox-hub internal.h, struct TargetLayer lists the block's weights: wqkv (the fused q / k / v
projection), wqkv_gate (the z projection), ssm_beta and ssm_alpha (per-token beta and alpha
projections) and ssm_out (the output projection after the delta net).  Readings taken here:
* a projection of rows x [M][K] by W [N][K] is y = x W^T: W holds one output feature per row with
  the input index fastest (the pages' [hidden, out] tensors, hidden fastest);
* beta = sigmoid(x W_beta^T), so that beta lies in (0, 1) as the delta rule takes it; alpha =
  x W_alpha^T, the softplus argument with dt_bias added by the layer;
* the block stores its intermediates as the layer's activation type: qkv, z, alpha, beta and the
  gated output are rounded to bf16 (round to nearest even) between the steps.
"""

from __future__ import annotations

import numpy as np

from oracle import ref


def linear(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """y[..., n] = sum_k x[..., k] w[n, k], in fp64."""
    return np.asarray(x, dtype=np.float64) @ np.asarray(w, dtype=np.float64).T


def sigmoid(x: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-np.asarray(x, dtype=np.float64)))


def bf16(x: np.ndarray) -> np.ndarray:
    """Round to the nearest bf16 (ties to even) through fp32, returned as fp64."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def in_projections(inp: dict) -> dict:
    """qkv, z, beta, alpha of the block, bf16-rounded."""
    x = inp["x"]
    return {"qkv": bf16(linear(x, inp["w_qkv"])), "z": bf16(linear(x, inp["w_z"])),
            "beta": bf16(sigmoid(linear(x, inp["w_beta"]))), "alpha": bf16(linear(x, inp["w_alpha"]))}


def block_verify(shape, inp: dict, flags: int = ref.F_QK_NORM_SILU) -> dict:
    """One GDN block step: the input projections, chain verify with capture (every drafted
    token), the output projection of the bf16 gated output.  Returns the verify's pool-level
    results plus 'proj' (the projections) and 'y' [B][T][hidden]."""
    proj = in_projections(inp)
    layer = dict(inp)
    B, T, Hv, dv = shape.n_batch, shape.n_tok, shape.n_vh, shape.d_v
    layer["qkv"] = proj["qkv"]
    layer["z"] = proj["z"].reshape(B, T, Hv, dv)
    layer["beta"] = proj["beta"]
    layer["alpha"] = proj["alpha"]
    r = ref.verify_pool(shape, layer, flags=flags)
    o = bf16(r["out"]).reshape(B, T, Hv * dv)
    r["proj"] = proj
    r["y"] = linear(o, inp["w_out"])
    return r
