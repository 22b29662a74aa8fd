"""Algorithmic HBM bytes and flops of each kernel: what the contract obliges a call to read and
write once (inputs, outputs, state, captures), not what any implementation happens to move.

Verify, per batch entry with a = activation bytes, o = output bytes, T tokens:
    T * (C*a + 2*H_v*a + H_v*d_v*(a + o))      qkv, alpha, beta, z in, out
  + 8 * H_v*d_v*d_k                            state read + write
  + 24 * C                                     conv state read + write (3 rows, fp32)
  + 4 * T * H_v*d_v*d_k                        per-position state capture
  + 4 * (3 + T) * C                            conv input window capture
  + 4                                          slot id
plus the parameters once: 4 * (2*H_v + 4*C + d_v).
"""

from __future__ import annotations

from .workloads import F32, Shape


def _ab(code: int) -> int:
    return 4 if code == F32 else 2


def params_bytes(s: Shape) -> int:
    return 4 * (2 * s.n_vh + 4 * s.conv_channels + s.d_v)


def verify_bytes(s: Shape, capture: bool = True, commit: bool = True) -> int:
    """Chain verify; commit=False is the deferred commit (GDN_F_DEFER_COMMIT), which reads the state
    and conv state but does not write them back."""
    a, o = _ab(s.act_dtype), _ab(s.out_dtype)
    C, Hv, dv, dk, T = s.conv_channels, s.n_vh, s.d_v, s.d_k, s.n_tok
    per = (T * (C * a + 2 * Hv * a + Hv * dv * (a + o)) + 8 * Hv * dv * dk + 24 * C + 4)
    if capture:
        per += 4 * T * Hv * dv * dk + 4 * (3 + T) * C
    if not commit:
        per -= 4 * Hv * dv * dk + 12 * C
    return s.n_batch * per + params_bytes(s)


def rollback_bytes(s: Shape, n: int) -> int:
    """Batched rollback of n slots: state and conv state copied (read + write) + indices."""
    per = 2 * 4 * (s.n_vh * s.d_v * s.d_k + 3 * s.conv_channels) + 8
    return n * per


def tree_bytes(s: Shape) -> int:
    """Tree verify lower bound: inputs, outputs, state and conv state read once, per-node state
    capture and per-node 3-row conv capture written once (no parent reloads counted)."""
    a, o = _ab(s.act_dtype), _ab(s.out_dtype)
    C, Hv, dv, dk, T = s.conv_channels, s.n_vh, s.d_v, s.d_k, s.n_tok
    per = (T * (C * a + 2 * Hv * a + Hv * dv * (a + o) + 4)  # + parent index
           + 4 * Hv * dv * dk + 12 * C + 4
           + 4 * T * Hv * dv * dk + 4 * T * 3 * C)
    return s.n_batch * per + params_bytes(s)


def prefill_bytes(s: Shape) -> int:
    """Chunked prefill of one slot: inputs and output once, state and conv state read + write."""
    a, o = _ab(s.act_dtype), _ab(s.out_dtype)
    C, Hv, dv, dk, T = s.conv_channels, s.n_vh, s.d_v, s.d_k, s.n_tok
    return (T * (C * a + 2 * Hv * a + Hv * dv * (a + o)) + 8 * Hv * dv * dk + 24 * C
            + params_bytes(s))


def verify_flops(s: Shape) -> int:
    """~7 d^2 flops per (slot, head, token) for the recurrence (S k, S q, rank-1 update with the
    decay) plus 8 per channel per token for the conv."""
    return s.n_batch * s.n_tok * (s.n_vh * 7 * s.d_v * s.d_k + 8 * s.conv_channels)


PREFILL_CHUNK = 64


def prefill_flops(s: Shape, chunk: int = PREFILL_CHUNK) -> int:
    """Dense products of the chunked (WY / UT) form, each counted once as 2 m n k, per token and
    value head: K K^T and Q K^T (2 C d_k each), T Y and P U (2 C d_v each), K S^T, Q S^T and the
    state update U^T K (2 d_k d_v each), plus the triangular inverse (C^2 / 3)."""
    C, dk, dv = chunk, s.d_k, s.d_v
    per_tok = 4 * C * dk + 4 * C * dv + 6 * dk * dv + (C * C) // 3
    return s.n_tok * s.n_vh * per_tok


def snapshot_bytes(s: Shape, n: int) -> int:
    """Snapshot or restore of n slots: state and conv state read from one buffer pair and written
    to the other."""
    return n * 2 * 4 * (s.n_vh * s.d_v * s.d_k + 3 * s.conv_channels)
