"""Device buffers for the verify path: torch owns the memory, libgdn computes.

Plumbing only: uploads the seeded inputs of ``workloads`` in the storage dtypes of include/gdn.h
and allocates outputs, capture buffers and workspaces with the documented shapes.
"""

from __future__ import annotations

from typing import Optional

import numpy as np
import torch

from . import gdn
from .workloads import BF16, Shape


def act_torch_dtype(code: int) -> torch.dtype:
    return torch.bfloat16 if code == BF16 else torch.float32


def upload(shape: Shape, inp: dict, *, device: str = "cuda", t_cap: Optional[int] = None,
           mode: int = gdn.GDN_CHAIN, capture: bool = True, fill_capture: float = float("nan"),
           flags: int = 0, eps: float = 1e-6) -> dict:
    """Device tensors for one call plus the ctypes dims / capture descriptors."""
    act = act_torch_dtype(shape.act_dtype)
    outd = act_torch_dtype(shape.out_dtype)
    B, T, P = shape.n_batch, shape.n_tok, shape.n_pool
    Hv, dv, dk, C = shape.n_vh, shape.d_v, shape.d_k, shape.conv_channels
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)
    d = {
        "qkv": f32(inp["qkv"]).to(act).contiguous(),
        "z": f32(inp["z"]).to(act).contiguous(),
        "alpha": f32(inp["alpha"]).to(act).contiguous(),
        "beta": f32(inp["beta"]).to(act).contiguous(),
        "A_log": f32(inp["A_log"]),
        "dt_bias": f32(inp["dt_bias"]),
        "conv_w": f32(inp["conv_w"]),
        "norm_w": f32(inp["norm_w"]),
        "state": f32(inp["state"]),
        "conv_state": f32(inp["conv_state"]),
        "slot_ids": torch.from_numpy(np.ascontiguousarray(inp["slot_ids"], dtype=np.int32)).to(device),
        # the prefill's slot, kept on the host so that a call does not read it back from the device
        "slot": int(np.asarray(inp["slot_ids"]).reshape(-1)[0]),
        "out": torch.empty((B, T, Hv, dv), dtype=outd, device=device),
    }
    if "parent" in inp:
        d["parent"] = torch.from_numpy(np.ascontiguousarray(inp["parent"], dtype=np.int32)).to(device)
    dims = gdn.make_dims(shape, flags=flags, eps=eps)
    d["dims"] = dims
    if capture:
        tc = T if t_cap is None else t_cap
        d["cap_ssm"] = torch.full((P, tc, Hv, dv, dk), fill_capture, dtype=torch.float32, device=device)
        conv_shape = (P, 3 + tc, C) if mode == gdn.GDN_CHAIN else (P, tc, 3, C)
        d["cap_conv"] = torch.full(conv_shape, fill_capture, dtype=torch.float32, device=device)
        d["capture"] = gdn.Capture(dims, d["cap_ssm"], d["cap_conv"], d["state"], d["conv_state"],
                                   tc, mode)
    return d


def verify(d: dict, n_batch: Optional[int] = None, stream=None, with_capture: bool = True) -> None:
    """gdn_verify over every token of the uploaded inputs (qkv is [B][T][C], so n_tok = T);
    ``n_batch`` may cut the batch to a prefix."""
    T = d["qkv"].shape[1]
    B = d["qkv"].shape[0] if n_batch is None else n_batch
    gdn.gdn_verify(d["dims"], d["state"], d["conv_state"], d["qkv"], d["z"], d["alpha"], d["beta"],
                   d["A_log"], d["dt_bias"], d["conv_w"], d["norm_w"],
                   d.get("capture") if with_capture else None, d["out"], T, d["slot_ids"], B,
                   stream)


def verify_resume(d: dict, resume_idx, n_batch: Optional[int] = None, stream=None, dims=None) -> None:
    """gdn_verify_resume over every token of the uploaded inputs: entry b starts from capture
    position resume_idx[b] (device int32) of the uploaded capture, or from its slot's state if < 0.
    ``dims`` replaces the uploaded dims (e.g. the same shape with other flags)."""
    T = d["qkv"].shape[1]
    B = d["qkv"].shape[0] if n_batch is None else n_batch
    gdn.gdn_verify_resume(d["dims"] if dims is None else dims, d["state"], d["conv_state"], d["qkv"], d["z"], d["alpha"],
                          d["beta"], d["A_log"], d["dt_bias"], d["conv_w"], d["norm_w"],
                          d["capture"], d["out"], T, d["slot_ids"], resume_idx, B, stream)


def verify_tree(d: dict, stream=None) -> None:
    B, T = d["parent"].shape
    gdn.gdn_verify_tree(d["dims"], d["state"], d["conv_state"], d["qkv"], d["z"], d["alpha"],
                        d["beta"], d["A_log"], d["dt_bias"], d["conv_w"], d["norm_w"], d["parent"],
                        d["capture"], d["out"], T, d["slot_ids"], B, stream)


def prefill(d: dict, stream=None) -> None:
    """gdn_prefill of every token of the uploaded single-entry inputs into slot slot_ids[0]."""
    T = d["qkv"].shape[1]
    need = gdn.gdn_prefill_workspace_bytes(d["dims"], T)
    ws = d.get("workspace")
    if ws is None or ws.numel() * 4 < need:
        ws = torch.empty((need + 3) // 4, dtype=torch.float32, device=d["qkv"].device)
        d["workspace"] = ws
    slot = d["slot"]
    gdn.gdn_prefill(d["dims"], d["state"], d["conv_state"], d["qkv"], d["z"], d["alpha"], d["beta"],
                    d["A_log"], d["dt_bias"], d["conv_w"], d["norm_w"], d["out"], T, slot, ws,
                    ws.numel() * 4, stream)


def snapshot_replay_round(d: dict, snap: dict, n_accept: int, stream=None) -> None:
    """One spec-decode round with snapshot-and-replay rollback on uploaded inputs (no capture):
    snapshot the batch's slots, verify all T tokens, and when n_accept < T restore the snapshot
    and verify the first n_accept tokens again.  snap holds pool-shaped "state" / "conv_state"."""
    B, T = d["qkv"].shape[0], d["qkv"].shape[1]
    gdn.gdn_snapshot(d["dims"], d["state"], d["conv_state"], snap["state"], snap["conv_state"], d["slot_ids"], B,
                     stream)
    verify(d, stream=stream, with_capture=False)
    if n_accept < T:
        gdn.gdn_restore(d["dims"], d["state"], d["conv_state"], snap["state"], snap["conv_state"], d["slot_ids"], B,
                        stream)
        rep = snap.get("replay")
        if rep is None or rep["n"] != n_accept:  # the accepted prefix of every input, contiguous
            rep = {"n": n_accept}
            for k in ("qkv", "z", "alpha", "beta"):
                rep[k] = d[k][:, :n_accept].contiguous()
            rep["out"] = d["out"][:, :n_accept].contiguous()
            snap["replay"] = rep
        gdn.gdn_verify(d["dims"], d["state"], d["conv_state"], rep["qkv"], rep["z"], rep["alpha"], rep["beta"],
                       d["A_log"], d["dt_bias"], d["conv_w"], d["norm_w"], None, rep["out"], n_accept,
                       d["slot_ids"], B, stream)


def layers_step(layers: list, slot_ids, accepted_idx, stream=None) -> None:
    """One spec-decode step over several layers, eagerly: gdn_verify of every layer (capture on,
    all uploaded tokens, every batch entry) with the shared slot_ids, then one
    gdn_rollback_layers to accepted_idx.  The launches a recorded gdn.Graph replays."""
    B, T = layers[0]["qkv"].shape[0], layers[0]["qkv"].shape[1]
    for d in layers:
        gdn.gdn_verify(d["dims"], d["state"], d["conv_state"], d["qkv"], d["z"], d["alpha"], d["beta"],
                       d["A_log"], d["dt_bias"], d["conv_w"], d["norm_w"], d["capture"], d["out"], T, slot_ids,
                       B, stream)
    gdn.gdn_rollback_layers([d["capture"] for d in layers], slot_ids, accepted_idx, B, stream)


def layers_graph(layers: list, slot_ids, accepted_idx,
                 phases: int = gdn.GDN_GRAPH_VERIFY | gdn.GDN_GRAPH_ROLLBACK) -> "gdn.Graph":
    """The same step recorded once (gdn_graph_create) over the uploaded layers' buffers."""
    B, T = layers[0]["qkv"].shape[0], layers[0]["qkv"].shape[1]
    return gdn.Graph(layers[0]["dims"], layers, layers[0]["capture"].t_cap, T, slot_ids, B, accepted_idx, phases)


def upload_block(shape: Shape, inp: dict, *, flags: int = gdn.GDN_F_QK_NORM_SILU) -> dict:
    """Device tensors of one GDN block call (workloads.make_block_inputs): the layer's buffers as
    upload() makes them (qkv, z, alpha, beta become outputs of the input projection), plus
    x [B*T][hidden], the concatenated input weight [C + H_v d_v + 2 H_v][hidden], w_out and
    y [B][T][hidden] (bf16)."""
    B, T, Hv, dv, C = shape.n_batch, shape.n_tok, shape.n_vh, shape.d_v, shape.conv_channels
    hidden = inp["x"].shape[-1]
    lay = dict(inp)
    lay.update(qkv=np.zeros((B, T, C), np.float32), z=np.zeros((B, T, Hv, dv), np.float32),
               alpha=np.zeros((B, T, Hv), np.float32), beta=np.zeros((B, T, Hv), np.float32))
    d = upload(shape, lay, flags=flags)
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda().to(torch.bfloat16).contiguous()
    d["x"] = bf(inp["x"].reshape(B * T, hidden))
    d["w_in"] = bf(np.concatenate([inp["w_qkv"], inp["w_z"], inp["w_beta"], inp["w_alpha"]], axis=0))
    d["w_out"] = bf(inp["w_out"])
    d["y"] = torch.empty((B, T, hidden), dtype=torch.bfloat16, device="cuda")
    d["hidden"] = hidden
    return d


def block_step(d: dict, stream=None) -> None:
    """One GDN block call: the four input projections as one gdn_linear (beta through a sigmoid),
    gdn_verify with capture over every token, the output projection of the gated output."""
    B, T, C = d["qkv"].shape
    Hv, dv = d["z"].shape[2], d["z"].shape[3]
    Z, hidden, M = Hv * dv, d["hidden"], B * T
    segs = [(0, C, d["qkv"], C, 0), (C, C + Z, d["z"], Z, 0),
            (C + Z, C + Z + Hv, d["beta"], Hv, 1), (C + Z + Hv, C + Z + 2 * Hv, d["alpha"], Hv, 0)]
    gdn.gdn_linear(d["x"], d["w_in"], M, C + Z + 2 * Hv, hidden, segs, stream)
    verify(d, stream=stream)
    gdn.gdn_linear(d["out"], d["w_out"], M, hidden, Z, [(0, hidden, d["y"], hidden, 0)], stream)
