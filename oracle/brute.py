"""Dense brute-force evaluation for tiny shapes (test infrastructure only).

An independent second route to the same definitions, used to pin the C oracle:

* conv: per channel, ``numpy.correlate`` of the extended input column with the 4 taps
  ('valid' mode), i.e. the textbook cross-correlation that a depthwise causal conv1d is;
* gate: ``-exp(A_log) * log(1 + exp(x))`` evaluated directly (fine for the small |x| of tests);
* update: the transition matrix rho * (I - beta k k^T) is formed explicitly as a d_k x d_k matrix
  and multiplied in, S <- S @ M + beta * outer(v, k) (gated delta rule, Yang, Kautz &
  Hatamizadeh 2024), no rank-1 shortcut;
* readout, norm and gate: o = S q, then the RMS norm and z * sigmoid(z) written out.

It shares no code with gdn_oracle.c.
"""

from __future__ import annotations

import numpy as np


def conv_brute(xext_col: np.ndarray, w: np.ndarray) -> np.ndarray:
    """Depthwise causal conv of one channel: xext_col has 3+T rows, w has 4 taps."""
    return np.correlate(np.asarray(xext_col, dtype=np.float64), np.asarray(w, dtype=np.float64),
                        mode="valid")


def chain_brute(shape, inp: dict, b: int, h: int, n_tok=None, flags: int = 0,
                eps: float = 1e-6) -> dict:
    """One (batch entry, value head) unit: states after every token, final state, o and y."""
    T = shape.n_tok if n_tok is None else int(n_tok)
    C = shape.conv_channels
    dk, dv = shape.d_k, shape.d_v
    r = shape.n_vh // shape.n_kh
    hk = h // r
    s = int(inp["slot_ids"][b])
    xext = np.concatenate([inp["conv_state"][s].astype(np.float64),
                           inp["qkv"][b, :T].astype(np.float64)], axis=0)
    xhat = np.empty((T, C))
    for c in range(C):
        xhat[:, c] = conv_brute(xext[:, c], inp["conv_w"][c])
    qs = xhat[:, hk * dk:(hk + 1) * dk]
    ks = xhat[:, shape.n_kh * dk + hk * dk: shape.n_kh * dk + (hk + 1) * dk]
    v0 = 2 * shape.n_kh * dk + h * dv
    vs = xhat[:, v0:v0 + dv]
    if flags & 1:
        silu = lambda x: x / (1.0 + np.exp(-x))
        qs, ks, vs = silu(qs), silu(ks), silu(vs)
        qs = qs / np.sqrt((qs ** 2).sum(-1, keepdims=True) + 1e-6) / np.sqrt(dk)
        ks = ks / np.sqrt((ks ** 2).sum(-1, keepdims=True) + 1e-6)
    S = inp["state"][s, h].astype(np.float64).copy()
    caps, os_, ys = [], [], []
    A = float(inp["A_log"][h])
    dtb = float(inp["dt_bias"][h])
    w = inp["norm_w"].astype(np.float64)
    for t in range(T):
        a = float(inp["alpha"][b, t, h])
        beta = float(inp["beta"][b, t, h])
        g = -np.exp(A) * np.log(1.0 + np.exp(a + dtb))
        rho = np.exp(g)
        k, v, q = ks[t], vs[t], qs[t]
        M = rho * (np.eye(dk) - beta * np.outer(k, k))
        S = S @ M + beta * np.outer(v, k)
        o = S @ q
        zt = inp["z"][b, t, h].astype(np.float64)
        y = o / np.sqrt(np.mean(o * o) + eps) * w * (zt / (1.0 + np.exp(-zt)))
        caps.append(S.copy())
        os_.append(o)
        ys.append(y)
    return {"state": S, "cap": np.array(caps), "o": np.array(os_), "y": np.array(ys),
            "xhat": xhat}
