"""GPU parity of the chunked (WY / UT) prefill against the sequential fp64 oracle."""

import numpy as np
import pytest

from gated_deltanet_linear_verify_amd import workloads as W
from oracle import ref
from tests.gpu_util import TOL_BF16, half_ulp_bf16, out_err, rel_err, say, to_np, tol_for

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_deltanet_linear_verify_amd import gdn
    gdn.lib()


def _mods():
    from gated_deltanet_linear_verify_amd import device, gdn
    return device, gdn


def _run_prefill(shape, inp, flags=0):
    device, gdn = _mods()
    d = device.upload(shape, inp, capture=False, flags=flags)
    device.prefill(d)
    torch.cuda.synchronize()
    return d


def _check(shape, inp, d, units=None, flags=0):
    o = ref.prefill_units(shape, inp, units, flags=flags)
    ub, uh = o["units"]
    s = int(inp["slot_ids"][0])
    st = to_np(d["state"])
    out = to_np(d["out"])
    ws, wo = 0.0, 0.0
    for u in range(len(ub)):
        h = int(uh[u])
        ws = max(ws, rel_err(st[s, h], o["state"][u]))
        wo = max(wo, out_err(shape, out[0, :, h], o["y"][u]))
    # conv state after the last token: a copy of the last three window rows
    win = ref.conv_window(shape, inp)
    np.testing.assert_array_equal(to_np(d["conv_state"])[s], win[0, -3:])
    say(f"  prefill {W.describe(shape)} worst rel err state {ws:.2e} out {wo:.2e}")
    tol = tol_for(shape)
    assert ws <= tol and wo <= tol


PREFILL_CASES = {
    # name: (shape, input kwargs, flags)
    "one_chunk_64": (W.shape_with(W.CHUNKED_PREFILL, n_tok=64), {}, 0),
    "ragged_100": (W.shape_with(W.CHUNKED_PREFILL, n_tok=100), {}, 0),
    "single_token": (W.shape_with(W.CHUNKED_PREFILL, n_tok=1), {}, 0),
    "two_tokens": (W.shape_with(W.CHUNKED_PREFILL, n_tok=2, n_pool=3), {}, 0),
    "weak_decay_640": (W.shape_with(W.CHUNKED_PREFILL, n_tok=640), {"weak_decay": True}, 0),
    "weak_decay_zero_state_333": (W.shape_with(W.CHUNKED_PREFILL, n_tok=333),
                                  {"weak_decay": True, "zero_state": True}, 0),
    "zero_state_256": (W.shape_with(W.CHUNKED_PREFILL, n_tok=256), {"zero_state": True}, 0),
    "fp32_d64_weak_200": (W.shape_with(W.TINY_VERIFY, n_tok=200, n_kh=2, n_vh=4),
                          {"weak_decay": True}, 0),
    "qk_norm_flag_160": (W.shape_with(W.CHUNKED_PREFILL, n_tok=160), {"weak_decay": True}, 1),
    "fp32_d128_weak_130": (W.shape_with(W.CHUNKED_PREFILL, n_tok=130, act_dtype=W.F32, out_dtype=W.F32),
                           {"weak_decay": True}, 0),
    "bf16_odd_heads_96": (W.shape_with(W.CHUNKED_PREFILL, n_tok=96, n_kh=3, n_vh=3), {"weak_decay": True}, 0),
    "bf16_d64_odd_heads_150": (W.shape_with(W.TINY_VERIFY, n_tok=150, n_kh=1, n_vh=3, act_dtype=W.BF16,
                                            out_dtype=W.BF16), {"weak_decay": True}, 0),
    # six value heads per key head: more than the prep keeps gates for at once (a second group)
    "bf16_d64_six_per_key_head_130": (W.shape_with(W.TINY_VERIFY, n_tok=130, n_kh=1, n_vh=6, act_dtype=W.BF16,
                                                   out_dtype=W.BF16), {"weak_decay": True}, 0),
    "bf16_d128_gqa4_70": (W.shape_with(W.CHUNKED_PREFILL, n_tok=70, n_kh=4, n_vh=16), {"weak_decay": True}, 0),
    # the q / k norm flag with fp32 activations at d = 128 (two conv passes over the channel halves)
    # and with bf16 at d = 64 (one pass)
    "fp32_d128_qk_norm_130": (W.shape_with(W.CHUNKED_PREFILL, n_tok=130, n_kh=2, n_vh=4, act_dtype=W.F32,
                                           out_dtype=W.F32), {"weak_decay": True}, 1),
    "bf16_d64_qk_norm_150": (W.shape_with(W.TINY_VERIFY, n_tok=150, n_kh=2, n_vh=4, act_dtype=W.BF16,
                                          out_dtype=W.BF16), {"weak_decay": True}, 1),
    # fp32 at the workloads' own decay (a 64-token chunk's running log decay reaches ~-90)
    "fp32_d128_standard_decay_130": (W.shape_with(W.CHUNKED_PREFILL, n_tok=130, n_kh=2, n_vh=4,
                                                  act_dtype=W.F32, out_dtype=W.F32), {}, 0),
}


@pytest.mark.parametrize("name", list(PREFILL_CASES))
def test_prefill_parity(name):
    shape, kw, flags = PREFILL_CASES[name]
    say(f"[prefill parity] {name}")
    inp = W.make_inputs(shape, 0, **kw)
    d = _run_prefill(shape, inp, flags)
    _check(shape, inp, d, flags=flags)


@pytest.mark.parametrize("base", ["bf16_d128", "fp32_d64", "bf16_d128_qk_norm"])
def test_prefill_extreme_gates(base):
    """alpha at -80 / +-30 / 20 (rho 1 to the last bit, or down to e^-82, so that the running decay
    of a 64-token chunk falls far below fp32's range), beta at 0 and 1 and z far into both SiLU
    tails, over four chunks with a ragged tail, against the sequential oracle at the usual bar."""
    shape = (W.shape_with(W.CHUNKED_PREFILL, n_tok=200) if base.startswith("bf16_d128")
             else W.shape_with(W.TINY_VERIFY, n_tok=200, n_kh=2, n_vh=4))
    flags = 1 if base.endswith("qk_norm") else 0  # SiLU after the conv, unit q / k, q / sqrt(d_k)
    say(f"[prefill extreme gates] {base}")
    inp = W.make_inputs(shape, 13)
    alpha = np.asarray(inp["alpha"]).copy()
    beta = np.asarray(inp["beta"]).copy()
    z = np.asarray(inp["z"]).copy()
    for t in range(shape.n_tok):
        alpha[:, t, :] = (-80.0, 30.0, -30.0, 0.0, 20.0)[t % 5]
        if t % 4 == 1:
            beta[:, t, :] = 0.0
        elif t % 4 == 3:
            beta[:, t, :] = 1.0
    z[:, ::3] = 20.0
    z[:, 1::3] *= -10.0
    # round the edits to the storage dtype, so that the device and the oracle read the same values
    act = shape.act_dtype
    inp.update(alpha=W.round_to(alpha, act), beta=W.round_to(beta, act), z=W.round_to(z, act))
    d = _run_prefill(shape, inp, flags=flags)
    _check(shape, inp, d, flags=flags)


def test_prefill_full_8192_every_head():
    """8192 tokens, 32 value heads: every head's final state and every token's output against the
    sequential oracle, for both the pages' decay and the weak-decay variant."""
    for kw in ({}, {"weak_decay": True}):
        shape = W.CHUNKED_PREFILL
        inp = W.make_inputs(shape, 0, **kw)
        d = _run_prefill(shape, inp)
        _check(shape, inp, d)


def test_prefill_matches_chain_verify():
    """The chunked form and the token-serial verify kernel agree (both against the oracle too)."""
    shape = W.shape_with(W.CHUNKED_PREFILL, n_tok=48)
    device, gdn = _mods()
    inp = W.make_inputs(shape, 4, weak_decay=True)
    p = _run_prefill(shape, inp)
    c = device.upload(shape, inp, capture=False)
    device.verify(c, with_capture=False)
    torch.cuda.synchronize()
    sp, sc = to_np(p["state"]), to_np(c["state"])
    assert rel_err(sp, sc) < 1e-4
    assert torch.equal(p["conv_state"], c["conv_state"])


def test_prefill_rejects_bad_arguments():
    device, gdn = _mods()
    shape = W.shape_with(W.CHUNKED_PREFILL, n_tok=64)
    inp = W.make_inputs(shape, 1)
    d = device.upload(shape, inp, capture=False)
    ws = torch.empty(16, dtype=torch.float32, device="cuda")
    with pytest.raises(gdn.GdnError) as ei:
        gdn.gdn_prefill(d["dims"], d["state"], d["conv_state"], d["qkv"], d["z"], d["alpha"],
                        d["beta"], d["A_log"], d["dt_bias"], d["conv_w"], d["norm_w"], d["out"], 64,
                        0, ws, 64)
    assert ei.value.code == gdn.GDN_ERR_ARG
    with pytest.raises(gdn.GdnError) as ei:
        device.prefill(dict(d, slot=5))
    assert ei.value.code == gdn.GDN_ERR_RANGE


def test_prefill_in_pieces_equals_one_call():
    """Prefilling 16 tokens per call (so every chunk has 16 tokens and the state crosses a call
    boundary every 16) agrees with one 160-token call (64-token chunks), and both with the oracle;
    the conv state, a plain copy of input rows, is identical."""
    device, gdn = _mods()
    shape = W.shape_with(W.CHUNKED_PREFILL, n_tok=160)
    inp = W.make_inputs(shape, 6, weak_decay=True)
    one = _run_prefill(shape, inp)
    _check(shape, inp, one)
    d = device.upload(shape, inp, capture=False)
    s = int(inp["slot_ids"][0])
    ws = torch.empty(gdn.gdn_prefill_workspace_bytes(d["dims"], 16) // 4, dtype=torch.float32,
                     device="cuda")
    for t0 in range(0, shape.n_tok, 16):
        sl = slice(t0, t0 + 16)
        gdn.gdn_prefill(d["dims"], d["state"], d["conv_state"], d["qkv"][:, sl], d["z"][:, sl],
                        d["alpha"][:, sl], d["beta"][:, sl], d["A_log"], d["dt_bias"], d["conv_w"],
                        d["norm_w"], d["out"][:, sl], 16, s, ws, ws.numel() * 4)
    torch.cuda.synchronize()
    _check(shape, inp, d)
    assert rel_err(to_np(d["state"][s]), to_np(one["state"][s])) < 1e-4
    # two bf16 outputs, each within half an ulp of its own fp32 value: allow one ulp between them
    a, b = to_np(d["out"]).astype(np.float64), to_np(one["out"]).astype(np.float64)
    gap = float(np.max(np.maximum(np.abs(a - b) - 2 * half_ulp_bf16(b), 0.0)) / np.max(np.abs(b)))
    assert gap < 1e-4, gap
    assert torch.equal(d["conv_state"], one["conv_state"])


def test_prefill_more_scan_workgroups_than_cus():
    """36 value heads: the scan's 288 workgroups (one per CU at most, by their LDS) exceed the CUs,
    so some start only when others have finished; held to the same bar."""
    shape = W.shape_with(W.CHUNKED_PREFILL, n_tok=100, n_kh=9, n_vh=36)
    say("[prefill parity] 36 heads, 288 scan workgroups")
    assert shape.n_vh * (shape.d_v // 16) > torch.cuda.get_device_properties(0).multi_processor_count
    inp = W.make_inputs(shape, 0, weak_decay=True)
    d = _run_prefill(shape, inp)
    _check(shape, inp, d)


def test_prefill_captured_in_a_graph_matches_eager():
    """The prefill recorded under stream capture: every replay of the graph, with eager work and
    synchronisation between replays, gives the eager call's output, state and conv state bit for
    bit (the same kernels on the same inputs)."""
    device, gdn = _mods()
    shape = W.shape_with(W.CHUNKED_PREFILL, n_tok=200)
    say("[prefill graph] 200 tokens, eager vs three replays")
    inp = W.make_inputs(shape, 3, weak_decay=True)
    d = device.upload(shape, inp, capture=False)
    st0, cs0 = d["state"].clone(), d["conv_state"].clone()
    device.prefill(d)
    torch.cuda.synchronize()
    _check(shape, inp, d)
    ref = [d["out"].clone(), d["state"].clone(), d["conv_state"].clone()]
    d["state"].copy_(st0)
    d["conv_state"].copy_(cs0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        device.prefill(d)
    for rep in range(3):
        d["state"].copy_(st0)
        d["conv_state"].copy_(cs0)
        d["out"].fill_(7.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(("out", "state", "conv_state"), (d["out"], d["state"], d["conv_state"]), ref):
            assert torch.equal(got, want), (rep, name)


def test_prefill_beta_zero_is_pure_decay():
    """beta = 0 and an identity conv (w = e_3): nothing is written, so S_t = exp(Gamma_t) S_0 and
    o_t = exp(Gamma_t) S_0 q_t with Gamma_t the running sum of g = -exp(A_log) softplus(alpha +
    dt_bias), checked against that closed form evaluated here in fp64."""
    shape = W.shape_with(W.CHUNKED_PREFILL, n_tok=200)
    inp = W.make_inputs(shape, 2, weak_decay=True)
    inp["beta"][:] = 0.0
    inp["conv_w"][:] = np.array([0.0, 0.0, 0.0, 1.0], dtype=np.float32)
    d = _run_prefill(shape, inp)
    T, Hv, Hk, dk = shape.n_tok, shape.n_vh, shape.n_kh, shape.d_k
    x = inp["alpha"][0].astype(np.float64) + inp["dt_bias"].astype(np.float64)[None, :]
    g = -np.exp(inp["A_log"].astype(np.float64))[None, :] * np.logaddexp(0.0, x)
    G = np.cumsum(g, axis=0)
    s = int(inp["slot_ids"][0])
    S0 = inp["state"][s].astype(np.float64)
    q = inp["qkv"][0, :, :Hk * dk].astype(np.float64).reshape(T, Hk, dk)
    z = inp["z"][0].astype(np.float64)
    w = inp["norm_w"].astype(np.float64)
    st, out = to_np(d["state"])[s], to_np(d["out"])[0]
    R = Hv // Hk
    ws_, wo_ = 0.0, 0.0
    for h in range(Hv):
        ws_ = max(ws_, rel_err(st[h], np.exp(G[-1, h]) * S0[h]))
        o = np.exp(G[:, h])[:, None] * (q[:, h // R] @ S0[h].T)
        y = o / np.sqrt(np.mean(o * o, axis=1, keepdims=True) + 1e-6) * w[None, :] \
            * (z[:, h] / (1.0 + np.exp(-z[:, h])))
        wo_ = max(wo_, out_err(shape, out[:, h], y))
    say(f"  beta = 0: worst rel err state {ws_:.2e} out {wo_:.2e}")
    assert ws_ <= TOL_BF16 and wo_ <= TOL_BF16
