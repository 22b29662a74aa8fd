"""Shared helpers of the GPU tests: comparison metrics and oracle-side assembly."""

import sys

import numpy as np

# Tolerances: max relative error per (slot, head) slice, ||gpu - ref||_inf / ||ref||_inf.
# All-fp32 inputs: 1e-5; bf16 inputs with fp32 state: 2e-3.  A bf16-stored output is held to the
# same budget after its own rounding is allowed for: rounding to bf16 (8 significant bits) moves
# a value by up to half an ulp, 2^-9 .. 2^-8 of itself, which alone can exceed 2e-3.
TOL_F32 = 1e-5
TOL_BF16 = 2e-3


def tol_for(shape):
    return TOL_F32 if shape.act_dtype == 0 else TOL_BF16


def rel_err(gpu, ref):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(gpu - ref)) / (den if den > 0 else 1.0))


def half_ulp_bf16(x):
    """Half a bf16 ulp at |x| (the largest error of round-to-nearest into bf16)."""
    ax = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    return np.where(ax > 0, np.exp2(e - 8), 0.0)


def rel_err_bf16_out(gpu, ref):
    """max(|gpu - ref| - half_ulp_bf16(ref), 0) / ||ref||_inf: the error left after the output's
    own bf16 rounding, relative to the slice's largest value."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.max(np.abs(ref))
    ex = np.maximum(np.abs(gpu - ref) - half_ulp_bf16(ref), 0.0)
    return float(np.max(ex) / (den if den > 0 else 1.0))


def out_err(shape, gpu, ref):
    return rel_err_bf16_out(gpu, ref) if shape.out_dtype == 1 else rel_err(gpu, ref)


def to_np(t):
    import torch
    return t.detach().to(torch.float32).cpu().numpy() if t.dtype != torch.int32 else t.cpu().numpy()


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rel_err_slices(gpu, ref, n_lead: int):
    """rel_err of every slice over the trailing axes, for arrays whose first n_lead axes index the
    slices (e.g. [units][T][d_v][d_k] with n_lead = 2: one value per unit and position)."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    ax = tuple(range(n_lead, ref.ndim))
    den = np.max(np.abs(ref), axis=ax)
    num = np.max(np.abs(gpu - ref), axis=ax)
    return num / np.where(den > 0, den, 1.0)


def out_err_slices(shape, gpu, ref, n_lead: int):
    """out_err of every slice over the trailing axes (bf16 outputs: beyond half an ulp of ref)."""
    if shape.out_dtype != 1:
        return rel_err_slices(gpu, ref, n_lead)
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    ax = tuple(range(n_lead, ref.ndim))
    den = np.max(np.abs(ref), axis=ax)
    ex = np.max(np.maximum(np.abs(gpu - ref) - half_ulp_bf16(ref), 0.0), axis=ax)
    return ex / np.where(den > 0, den, 1.0)
