"""Pins of the CPU oracle against things other than itself.

Each test fixes one part of the definition so that a plausible slip in the oracle (a dropped
term, a wrong sign, a transposed operand, an off-by-one index) fails at least one of them:
exact rational brute force, dense numpy brute force, closed forms, invariants, library
routines and the indexing contract printed on the pages.
"""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from gated_deltanet_linear_verify_amd import workloads as W
from oracle import brute, ref

HERE = os.path.dirname(os.path.abspath(__file__))

TINY = W.shape_with(W.TINY_VERIFY, d_k=8, d_v=8, n_kh=2, n_vh=4, n_tok=5, n_pool=3, n_batch=2)


def _identity_conv(inp, shape):
    w = np.zeros((shape.conv_channels, 4), dtype=np.float32)
    w[:, 3] = 1.0
    inp["conv_w"] = w


def _rel(a, b):
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)


# ---------------------------------------------------------------- dense brute force -------

@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("flags", [0, 1])
def test_oracle_matches_dense_brute_force(seed, flags):
    """C oracle (expanded rank-1 form) == numpy dense (I - beta k k^T) product form."""
    inp = W.make_inputs(TINY, seed)
    r = ref.verify_units(TINY, inp, flags=flags, want_o=True)
    ub, uh = r["units"]
    for u in range(len(ub)):
        bf = brute.chain_brute(TINY, inp, int(ub[u]), int(uh[u]), flags=flags)
        assert _rel(r["cap"][u], bf["cap"]) < 1e-12
        assert _rel(r["state"][u], bf["state"]) < 1e-12
        assert _rel(r["o"][u], bf["o"]) < 1e-12
        assert _rel(r["y"][u], bf["y"]) < 1e-12


def test_conv_matches_numpy_correlate():
    """The conv is per-channel cross-correlation ('valid') of concat(conv_state, qkv)."""
    inp = W.make_inputs(TINY, 3)
    win = ref.conv_window(TINY, inp)
    for b in range(TINY.n_batch):
        xhat = ref.conv(TINY, inp, b)
        for c in range(TINY.conv_channels):
            expect = np.correlate(win[b, :, c].astype(np.float64),
                                  inp["conv_w"][c].astype(np.float64), mode="valid")
            np.testing.assert_allclose(xhat[:, c], expect, rtol=1e-14, atol=1e-15)


def test_conv_one_hot_taps():
    """Tap 3 is the current token (identity); tap 0 is a delay of three rows that reads the
    slot's conv state for the first three tokens."""
    shape = TINY
    inp = W.make_inputs(shape, 4)
    _identity_conv(inp, shape)
    for b in range(shape.n_batch):
        np.testing.assert_array_equal(ref.conv(shape, inp, b), inp["qkv"][b].astype(np.float64))
    w0 = np.zeros_like(inp["conv_w"])
    w0[:, 0] = 1.0
    inp["conv_w"] = w0
    for b in range(shape.n_batch):
        s = int(inp["slot_ids"][b])
        xhat = ref.conv(shape, inp, b)
        np.testing.assert_array_equal(xhat[:3], inp["conv_state"][s].astype(np.float64))
        np.testing.assert_array_equal(xhat[3:], inp["qkv"][b, :shape.n_tok - 3].astype(np.float64))


# ---------------------------------------------------------------- exact rational ---------

def _fraction_chain(S0, ks, vs, qs, betas):
    """Exact S_t = S_{t-1} (I - beta k k^T) + beta v k^T (rho = 1) and o_t = S_t q_t."""
    d = len(S0)
    S = [row[:] for row in S0]
    caps, outs = [], []
    for k, v, q, b in zip(ks, vs, qs, betas):
        M = [[(Fraction(1) if i == j else Fraction(0)) - b * k[i] * k[j] for j in range(d)]
             for i in range(d)]
        S = [[sum(S[i][m] * M[m][j] for m in range(d)) + b * v[i] * k[j] for j in range(d)]
             for i in range(d)]
        caps.append([row[:] for row in S])
        outs.append([sum(S[i][j] * q[j] for j in range(d)) for i in range(d)])
    return caps, outs


def test_exact_rational_brute_force():
    """rho = 1 (A_log = -inf makes g = -0), identity conv, dyadic inputs: the oracle must agree
    with exact rational arithmetic to the last few ulps."""
    d = 4
    shape = W.shape_with(TINY, d_k=d, d_v=d, n_kh=1, n_vh=1, n_tok=3, n_pool=1, n_batch=1,
                         act_dtype=W.F32)
    rng = np.random.default_rng(7)
    dy = lambda n: (rng.integers(-8, 9, size=n) / 8.0)
    inp = W.make_inputs(shape, 0)
    _identity_conv(inp, shape)
    inp["qkv"] = dy(inp["qkv"].size).reshape(inp["qkv"].shape).astype(np.float32)
    inp["state"] = dy(inp["state"].size).reshape(inp["state"].shape).astype(np.float32)
    inp["beta"] = np.array([[[0.5], [0.25], [0.75]]], dtype=np.float32)
    inp["A_log"] = np.array([-np.inf], dtype=np.float32)
    r = ref.verify_units(shape, inp, want_o=True)
    assert r["cap"].shape == (1, 3, d, d)
    F = lambda x: Fraction(float(x))
    S0 = [[F(x) for x in row] for row in inp["state"][0, 0]]
    ks = [[F(x) for x in inp["qkv"][0, t, d:2 * d]] for t in range(3)]
    qs = [[F(x) for x in inp["qkv"][0, t, 0:d]] for t in range(3)]
    vs = [[F(x) for x in inp["qkv"][0, t, 2 * d:3 * d]] for t in range(3)]
    bs = [F(x) for x in inp["beta"][0, :, 0]]
    caps, outs = _fraction_chain(S0, ks, vs, qs, bs)
    exact_cap = np.array([[[float(x) for x in row] for row in c] for c in caps])
    exact_o = np.array([[float(x) for x in o] for o in outs])
    assert np.max(np.abs(r["cap"][0] - exact_cap)) <= 1e-14 * max(1.0, np.max(np.abs(exact_cap)))
    assert np.max(np.abs(r["o"][0] - exact_o)) <= 1e-14 * max(1.0, np.max(np.abs(exact_o)))


# ---------------------------------------------------------------- closed forms -----------

def test_one_token_from_zero_state():
    """S_0 = 0: S_1 = beta v k^T and o_1 = beta (k . q) v, whatever the decay."""
    shape = W.shape_with(TINY, n_tok=1)
    inp = W.make_inputs(shape, 5, zero_state=True)
    _identity_conv(inp, shape)
    r = ref.verify_units(shape, inp, want_o=True)
    ub, uh = r["units"]
    r_ = shape.n_vh // shape.n_kh
    dk = shape.d_k
    for u in range(len(ub)):
        b, h = int(ub[u]), int(uh[u])
        hk = h // r_
        x = inp["qkv"][b, 0].astype(np.float64)
        q = x[hk * dk:(hk + 1) * dk]
        k = x[shape.n_kh * dk + hk * dk: shape.n_kh * dk + (hk + 1) * dk]
        v = x[2 * shape.n_kh * dk + h * shape.d_v: 2 * shape.n_kh * dk + (h + 1) * shape.d_v]
        beta = float(inp["beta"][b, 0, h])
        np.testing.assert_allclose(r["state"][u], beta * np.outer(v, k), rtol=1e-13, atol=1e-16)
        np.testing.assert_allclose(r["o"][u, 0], beta * np.dot(k, q) * v, rtol=1e-12, atol=1e-15)


def test_beta_zero_and_no_decay_is_identity_bit_exact():
    """beta = 0 and g = 0 (alpha = -1e30 makes softplus exactly 0) leave the state unchanged."""
    inp = W.make_inputs(TINY, 6)
    inp["beta"][:] = 0.0
    inp["alpha"][:] = -1e30
    assert ref.gate(inp["A_log"][0], inp["dt_bias"][0], -1e30) == 0.0
    r = ref.verify_units(TINY, inp)
    ub, uh = r["units"]
    for u in range(len(ub)):
        s = int(inp["slot_ids"][ub[u]])
        S0 = inp["state"][s, uh[u]].astype(np.float64)
        np.testing.assert_array_equal(r["state"][u], S0)
        for t in range(TINY.n_tok):
            np.testing.assert_array_equal(r["cap"][u, t], S0)


def test_pure_decay_closed_form():
    """beta = 0: o_t = exp(Gamma_t) S_0 q_t with Gamma_t the running sum of
    g = -exp(A_log) * log(1 + exp(alpha + dt_bias)) (numpy logaddexp as the library softplus)."""
    shape = W.shape_with(TINY, n_tok=12)
    inp = W.make_inputs(shape, 8, weak_decay=True)
    inp["beta"][:] = 0.0
    r = ref.verify_units(shape, inp, want_o=True)
    ub, uh = r["units"]
    for u in range(len(ub)):
        b, h = int(ub[u]), int(uh[u])
        s = int(inp["slot_ids"][b])
        xhat = ref.conv(shape, inp, b)
        hk = h // (shape.n_vh // shape.n_kh)
        g = -np.exp(np.float64(inp["A_log"][h])) * np.logaddexp(
            0.0, inp["alpha"][b, :, h].astype(np.float64) + np.float64(inp["dt_bias"][h]))
        gam = np.cumsum(g)
        S0 = inp["state"][s, h].astype(np.float64)
        for t in range(shape.n_tok):
            q = xhat[t, hk * shape.d_k:(hk + 1) * shape.d_k]
            np.testing.assert_allclose(r["o"][u, t], np.exp(gam[t]) * (S0 @ q), rtol=1e-11,
                                       atol=1e-14)


def test_delta_rule_write_property():
    """beta = 1, g = 0 and |k| = 1 exactly: after the update S_t k_t = v_t (the delta rule
    overwrites the value stored at key k).  A non-symmetric start state pins the orientation
    of S (a transposed state would read S^T k instead)."""
    shape = W.shape_with(TINY, n_tok=6, act_dtype=W.F32)
    inp = W.make_inputs(shape, 9)
    _identity_conv(inp, shape)
    rng = np.random.default_rng(19)
    dk = shape.d_k
    k0 = shape.n_kh * dk
    for b in range(shape.n_batch):
        for t in range(shape.n_tok):
            for hk in range(shape.n_kh):
                k = np.zeros(dk, dtype=np.float32)
                idx = rng.choice(dk, size=4, replace=False)
                k[idx] = 0.5 * rng.choice([-1.0, 1.0], size=4)
                inp["qkv"][b, t, k0 + hk * dk:k0 + (hk + 1) * dk] = k
    inp["beta"][:] = 1.0
    inp["alpha"][:] = -1e30
    S = inp["state"]
    assert np.max(np.abs(S[0, 0] - S[0, 0].T)) > 1e-2
    r = ref.verify_units(shape, inp)
    ub, uh = r["units"]
    for u in range(len(ub)):
        b, h = int(ub[u]), int(uh[u])
        hk = h // (shape.n_vh // shape.n_kh)
        for t in range(shape.n_tok):
            x = inp["qkv"][b, t].astype(np.float64)
            k = x[k0 + hk * dk:k0 + (hk + 1) * dk]
            v = x[2 * k0 + h * shape.d_v:2 * k0 + (h + 1) * shape.d_v]
            assert np.dot(k, k) == 1.0
            np.testing.assert_allclose(r["cap"][u, t] @ k, v, rtol=0, atol=1e-14)


def test_scalar_recurrence_by_hand():
    """d_k = d_v = 1: s_t = rho s (1 - beta k^2) + beta v k, evaluated here by hand."""
    shape = W.shape_with(TINY, d_k=1, d_v=1, n_kh=1, n_vh=1, n_tok=3, n_pool=1, n_batch=1,
                         act_dtype=W.F32)
    inp = W.make_inputs(shape, 0)
    _identity_conv(inp, shape)
    inp["qkv"] = np.array([[[0.5, 2.0, 3.0], [1.0, -1.0, 0.5], [2.0, 0.25, -4.0]]],
                          dtype=np.float32)  # q, k, v per token
    inp["state"] = np.array([[[[0.75]]]], dtype=np.float32)
    inp["beta"] = np.array([[[0.5], [1.0], [0.25]]], dtype=np.float32)
    inp["A_log"] = np.array([0.0], dtype=np.float32)
    inp["dt_bias"] = np.array([0.0], dtype=np.float32)
    inp["alpha"] = np.array([[[0.0], [1.0], [-2.0]]], dtype=np.float32)
    r = ref.verify_units(shape, inp, want_o=True)
    s = 0.75
    # g = -exp(0) * ln(1 + e^alpha)
    rhos = [1.0 / (1.0 + math.exp(a)) for a in (0.0, 1.0, -2.0)]  # exp(-ln(1+e^a))
    toks = [(0.5, 2.0, 3.0, 0.5), (1.0, -1.0, 0.5, 1.0), (2.0, 0.25, -4.0, 0.25)]
    for t, ((q, k, v, b), rho) in enumerate(zip(toks, rhos)):
        s = rho * s * (1.0 - b * k * k) + b * v * k
        assert abs(r["cap"][0, t, 0, 0] - s) < 1e-14
        assert abs(r["o"][0, t, 0] - s * q) < 1e-14


# ---------------------------------------------------------------- gate / norm ------------

@pytest.mark.parametrize("x", [-60.0, -5.0, -0.5, 0.0, 0.3, 4.0, 35.0, 300.0])
def test_gate_against_library_softplus(x):
    """g = -exp(A_log) * softplus(x) with softplus from numpy's logaddexp; softplus(0) = ln 2."""
    for A in (-3.0, 0.0, 0.7):
        g = ref.gate(A, 0.0, x)
        expect = -math.exp(A) * float(np.logaddexp(0.0, x))
        assert g == pytest.approx(expect, rel=1e-14, abs=1e-300)
        assert g <= 0.0
    assert ref.softplus(0.0) == pytest.approx(math.log(2.0), rel=1e-15)


def test_norm_gate_against_torch_rms_norm():
    import torch
    import torch.nn.functional as Fn

    rng = np.random.default_rng(11)
    for n in (1, 7, 64, 128):
        o = rng.standard_normal(n)
        z = rng.standard_normal(n).astype(np.float32)
        w = (1 + 0.1 * rng.standard_normal(n)).astype(np.float32)
        y = ref.norm_gate(o, z, w, 1e-6)
        ot = torch.from_numpy(o)
        expect = (Fn.rms_norm(ot, (n,), torch.from_numpy(w.astype(np.float64)), 1e-6)
                  * Fn.silu(torch.from_numpy(z.astype(np.float64)))).numpy()
        np.testing.assert_allclose(y, expect, rtol=1e-13, atol=1e-15)
        # invariant: rms of y / (w silu(z)) is sqrt(m / (m + eps)), m = mean(o^2)
        m = np.mean(o * o)
        z64, w64 = z.astype(np.float64), w.astype(np.float64)
        ratio = y / (w64 * z64 / (1 + np.exp(-z64)))
        assert math.sqrt(np.mean(ratio ** 2)) == pytest.approx(math.sqrt(m / (m + 1e-6)),
                                                                rel=1e-12)


def test_gqa_map_key_head_reaches_its_value_heads_only():
    """Changing key head j's k channels changes exactly value heads j*r .. j*r + r - 1."""
    shape = TINY
    r_ = shape.n_vh // shape.n_kh
    inp = W.make_inputs(shape, 12)
    base = ref.verify_units(shape, inp)
    for j in range(shape.n_kh):
        inp2 = {k: v.copy() for k, v in inp.items()}
        k0 = shape.n_kh * shape.d_k + j * shape.d_k
        inp2["qkv"][:, :, k0:k0 + shape.d_k] *= -0.5
        r2 = ref.verify_units(shape, inp2)
        ub, uh = base["units"]
        for u in range(len(ub)):
            changed = not np.array_equal(base["state"][u], r2["state"][u])
            assert changed == (int(uh[u]) // r_ == j), (u, j)


# ---------------------------------------------------------------- capture / rollback -----

def test_rollback_indexing_golden():
    """The accepted index and conv rows printed by the rollback contract."""
    with open(os.path.join(HERE, "golden", "rollback_indexing.json")) as f:
        g = json.load(f)
    K = g["kernel"]
    for c in g["cases"]:
        a = ref.accepted_index(c["n_tokens_max"], c["trim"])
        assert a == c["accepted_idx"], c
        if a is not None:
            commit_n = a + 1
            assert list(range(commit_n, commit_n + K - 1)) == c["conv_rows"]


def _tagged_window_inputs(n_tok: int) -> tuple:
    """A tiny call whose conv input window rows are tagged: row r of concat(conv state, qkv) holds
    the value 1000 r + channel index in every channel, so a restored or advanced conv state names
    the rows it came from."""
    shape = W.shape_with(TINY, n_tok=n_tok, n_pool=3, n_batch=1)
    inp = W.make_inputs(shape, 40)
    C = shape.conv_channels
    s = int(inp["slot_ids"][0])
    row = lambda r: (1000.0 * r + np.arange(C)).astype(np.float32)
    inp["conv_state"][s] = np.stack([row(r) for r in range(3)])
    inp["qkv"][0] = np.stack([row(3 + t) for t in range(n_tok)])
    return shape, inp, s, row


@pytest.mark.parametrize("case", [c for c in json.load(open(os.path.join(HERE, "golden", "rollback_indexing.json")))["cases"]
                                  if c["accepted_idx"] is not None])
def test_rollback_indexing_golden_through_the_oracle(case):
    """The golden conv rows, through the oracle's own rollback and its verify: after verifying
    n_tokens_max tokens, ref.rollback_chain to the golden accepted index restores exactly the golden
    window rows as the conv state, and so does the final conv state of a verify of the accepted
    tokens alone (commit_n = accepted_idx + 1 tokens); the restored recurrent state is capture
    element accepted_idx, which equals that shorter verify's state."""
    n, a = case["n_tokens_max"], case["accepted_idx"]
    shape, inp, s, row = _tagged_window_inputs(n)
    full = ref.verify_pool(shape, inp)
    st = inp["state"].astype(np.float64).copy()
    cs = inp["conv_state"].copy()
    ref.rollback_chain(st, cs, full["cap_ssm"], full["cap_conv"], s, a)
    want = np.stack([row(r) for r in case["conv_rows"]])
    np.testing.assert_array_equal(cs[s], want)
    short = ref.verify_pool(shape, inp, n_tok=a + 1)
    np.testing.assert_array_equal(short["conv_state"][s], want)
    np.testing.assert_array_equal(st[s], short["state"][s])
    # a verify of all n_tokens_max tokens ends on the rows after the last one
    np.testing.assert_array_equal(full["conv_state"][s], np.stack([row(r) for r in range(n, n + 3)]))


@pytest.mark.parametrize("shape_name", ["tiny_verify", "small"])
def test_verify_then_rollback_equals_shorter_verify(shape_name):
    """verify(T) then rollback(a) leaves exactly what verify(a + 1) leaves (state and conv
    state), for every accepted index a."""
    shape = W.TINY_VERIFY if shape_name == "tiny_verify" else TINY
    inp = W.make_inputs(shape, 13)
    full = ref.verify_pool(shape, inp)
    for a in range(shape.n_tok):
        st = inp["state"].astype(np.float64).copy()
        cs = inp["conv_state"].copy()
        for b in range(shape.n_batch):
            s = int(inp["slot_ids"][b])
            ref.rollback_chain(st, cs, full["cap_ssm"], full["cap_conv"], s, a)
        short = ref.verify_pool(shape, inp, n_tok=a + 1)
        np.testing.assert_array_equal(st, short["state"])
        np.testing.assert_array_equal(cs, short["conv_state"])
    # the last position's capture is the advanced state (trim 0 is a no-op)
    for b in range(shape.n_batch):
        s = int(inp["slot_ids"][b])
        np.testing.assert_array_equal(full["cap_ssm"][s, -1], full["state"][s])


def test_untouched_slots_keep_their_state():
    shape = W.shape_with(TINY, n_pool=5, n_batch=2)
    inp = W.make_inputs(shape, 14)
    full = ref.verify_pool(shape, inp)
    used = set(int(s) for s in inp["slot_ids"])
    for s in range(shape.n_pool):
        if s not in used:
            np.testing.assert_array_equal(full["state"][s], inp["state"][s].astype(np.float64))
            np.testing.assert_array_equal(full["conv_state"][s], inp["conv_state"][s])


def test_slot_permutation_invariance():
    """Per-slot results do not depend on which batch entry carries the slot."""
    shape = W.shape_with(TINY, n_pool=3, n_batch=3)
    inp = W.make_inputs(shape, 15)
    a = ref.verify_pool(shape, inp)
    perm = np.array([2, 0, 1])
    inp2 = dict(inp)
    for k in ("qkv", "z", "alpha", "beta"):
        inp2[k] = inp[k][perm]
    inp2["slot_ids"] = inp["slot_ids"][perm]
    b = ref.verify_pool(shape, inp2)
    np.testing.assert_array_equal(a["state"], b["state"])
    np.testing.assert_array_equal(a["conv_state"], b["conv_state"])
    np.testing.assert_array_equal(a["out"][perm], b["out"])


# ---------------------------------------------------------------- tree -------------------

def _gather_path(shape, inp, b, path):
    """Inputs of a single-entry chain made of the tokens on a root path."""
    sub = W.shape_with(shape, n_tok=len(path), n_batch=1)
    d = {k: v for k, v in inp.items()}
    for k in ("qkv", "z", "alpha", "beta"):
        d[k] = inp[k][b:b + 1, path]
    d["slot_ids"] = inp["slot_ids"][b:b + 1]
    return sub, d


def test_tree_node_equals_chain_of_root_path_brute_force():
    shape = W.shape_with(TINY, n_tok=10, n_batch=2, n_pool=3)
    inp = W.make_tree_inputs(shape, 16)
    rng = np.random.default_rng(3)
    inp["parent"] = np.stack([W.random_tree(rng, shape.n_tok, 3) for _ in range(2)])
    r = ref.tree_units(shape, inp)
    cc = ref.tree_conv(shape, inp)
    ub, uh = r["units"]
    for u in range(len(ub)):
        b, h = int(ub[u]), int(uh[u])
        for i in range(shape.n_tok):
            path = []
            n = i
            while n >= 0:
                path.append(n)
                n = int(inp["parent"][b, n])
            path.reverse()
            sub, d = _gather_path(shape, inp, b, path)
            bf = brute.chain_brute(sub, d, 0, h)
            assert _rel(r["cap"][u, i], bf["state"]) < 1e-12
            assert _rel(r["y"][u, i], bf["y"][-1]) < 1e-12
            if h == 0:
                win = np.concatenate([inp["conv_state"][int(inp["slot_ids"][b])],
                                      inp["qkv"][b, path]], axis=0)
                np.testing.assert_array_equal(cc[b, i], win[-3:])


def test_tree_with_chain_parents_equals_chain():
    shape = W.shape_with(TINY, n_tok=7)
    inp = W.make_inputs(shape, 17)
    inp["parent"] = np.stack([W.chain_parents(shape.n_tok)] * shape.n_batch)
    t = ref.tree_units(shape, inp)
    c = ref.verify_units(shape, inp)
    np.testing.assert_array_equal(t["cap"], c["cap"])
    np.testing.assert_array_equal(t["y"], c["y"])
    cc = ref.tree_conv(shape, inp)
    win = ref.conv_window(shape, inp)
    for i in range(shape.n_tok):
        np.testing.assert_array_equal(cc[:, i], win[:, i + 1:i + 4])


def test_tree_rejects_malformed_parents():
    shape = W.shape_with(TINY, n_tok=4)
    inp = W.make_inputs(shape, 18)
    inp["parent"] = np.array([[-1, 0, 2, 1]] * shape.n_batch, dtype=np.int32)
    with pytest.raises(ValueError):
        ref.tree_units(shape, inp)


# ---------------------------------------------------------------- the block's projections

def test_linear_equals_integer_brute_force():
    """x W^T on small integer matrices (exact in fp64) against a pure-Python triple loop; the
    shapes are all different, so a transposed operand cannot pass."""
    from oracle import block
    rng = np.random.default_rng(3)
    x = rng.integers(-9, 10, (3, 5))
    w = rng.integers(-9, 10, (4, 5))
    want = [[sum(int(x[m, k]) * int(w[n, k]) for k in range(5)) for n in range(4)] for m in range(3)]
    assert np.array_equal(block.linear(x, w), np.array(want, dtype=np.float64))


def test_linear_identity_and_sigmoid():
    from scipy.special import expit
    from oracle import block
    w = np.arange(12.0).reshape(3, 4)
    assert np.array_equal(block.linear(np.eye(4), w), w.T)  # unit rows pick out the weights' columns
    xs = np.linspace(-30, 30, 121)
    np.testing.assert_allclose(block.sigmoid(xs), expit(xs), rtol=1e-15, atol=0)
    assert block.sigmoid(np.array([0.0]))[0] == 0.5


def test_bf16_rounding_against_torch():
    """The oracle's own round-to-nearest-even bf16 against torch's conversion, ties included."""
    import torch
    from oracle import block
    rng = np.random.default_rng(4)
    x = np.concatenate([rng.standard_normal(4096) * 10.0 ** rng.integers(-6, 6, 4096),
                        np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8), 0.0])])
    want = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(block.bf16(x), want.astype(np.float64))
    assert block.bf16(np.array([1.0 + 2.0 ** -8]))[0] == 1.0           # tie, to even
    assert block.bf16(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 1.0 + 2.0 ** -6  # tie, to even


def test_block_composes_its_parts():
    """With unit rows as x the projections return chosen columns of the weights, so the block
    must equal the chain verify of those exact activations followed by the output projection."""
    from oracle import block
    shape = W.shape_with(TINY, act_dtype=W.BF16, out_dtype=W.BF16, n_tok=2, n_batch=1, n_pool=1)
    B, T, Hv, dv, C = shape.n_batch, shape.n_tok, shape.n_vh, shape.d_v, shape.conv_channels
    hidden = B * T
    inp = W.make_block_inputs(shape, hidden, seed=5)
    inp["x"] = np.eye(hidden).reshape(B, T, hidden)
    plain = W.make_inputs(shape, 5)
    # choose the weights so that the projections reproduce plain's activations
    inp["w_qkv"] = plain["qkv"].reshape(hidden, C).T.astype(np.float64)
    inp["w_z"] = plain["z"].reshape(hidden, Hv * dv).T.astype(np.float64)
    inp["w_alpha"] = plain["alpha"].reshape(hidden, Hv).T.astype(np.float64)
    logit = np.log(plain["beta"] / (1.0 - plain["beta"]))  # sigmoid(logit) = beta
    inp["w_beta"] = logit.reshape(hidden, Hv).T
    r = block.block_verify(shape, inp, flags=0)
    want = ref.verify_pool(shape, plain, flags=0)
    np.testing.assert_allclose(r["proj"]["beta"].reshape(plain["beta"].shape), plain["beta"], rtol=4e-3)
    lay = dict(plain)
    lay["beta"] = r["proj"]["beta"].reshape(plain["beta"].shape)
    want = ref.verify_pool(shape, lay, flags=0)
    assert np.array_equal(r["state"], want["state"])
    y = block.linear(block.bf16(want["out"]).reshape(B, T, Hv * dv), inp["w_out"])
    assert np.array_equal(r["y"], y)
