"""GPU parity of gdn_verify_resume: a verify that starts each entry from a capture position of the
previous round (its rollback folded into the state load), against gdn_rollback_batch + gdn_verify
bit for bit and against the oracle run from the restored state (through the C ABI)."""

import numpy as np
import pytest

from gated_deltanet_linear_verify_amd import workloads as W
from oracle import ref
from tests.gpu_util import out_err, rel_err, say, to_np, tol_for

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_deltanet_linear_verify_amd import gdn
    gdn.lib()  # fail loudly if the HIP library is missing


def _dev():
    from gated_deltanet_linear_verify_amd import device
    return device


def _gdn():
    from gated_deltanet_linear_verify_amd import gdn
    return gdn


ACTS = ("qkv", "z", "alpha", "beta")


def _next_round(d, inp2):
    """Load the second round's activations into the uploaded buffers (state and capture stay)."""
    for k in ACTS:
        src = torch.from_numpy(np.ascontiguousarray(inp2[k], dtype=np.float32)).to(d[k].device)
        d[k].copy_(src.to(d[k].dtype))


def _snapshot(d, T):
    return {"state": to_np(d["state"]), "conv_state": to_np(d["conv_state"]),
            "out": to_np(d["out"].float()), "cap_ssm": to_np(d["cap_ssm"][:, :T]),
            "cap_conv": to_np(d["cap_conv"][:, :3 + T])}


def _accepted(shape, inp, rng, with_fresh=True):
    """Per-entry accepted position of the first verify round (K - trim); with_fresh marks a few entries -1 (start
    from the slot's state, as after a fully accepted round that was already committed)."""
    K = shape.n_tok - 1
    acc = np.array([K - int(t) for t in inp["trims"]], dtype=np.int32)
    if with_fresh and shape.n_batch > 1:
        acc[rng.choice(shape.n_batch, size=max(1, shape.n_batch // 4), replace=False)] = -1
    return acc


RESUME_CASES = {
    # name: (shape, seed of the first verify round, seed of the second)
    "tiny_fp32": (W.shape_with(W.TINY_VERIFY, n_pool=4, n_batch=3), 0, 1),
    "bf16_d128_ten_slots": (W.shape_with(W.MULTI_SLOT_VERIFY, n_pool=12, n_batch=10), 7, 8),
    "bf16_three_launches_37": (W.shape_with(W.SINGLE_SLOT_VERIFY, n_tok=37, n_pool=3, n_batch=2), 3, 4),
    "bf16_gqa4_one_token": (W.shape_with(W.SINGLE_SLOT_VERIFY, n_kh=4, n_vh=16, n_tok=1, n_pool=3, n_batch=3),
                            5, 6),
}


@pytest.mark.parametrize("name", list(RESUME_CASES))
def test_resume_equals_rollback_then_verify_bitwise(name):
    shape, s1, s2 = RESUME_CASES[name]
    say(f"[resume == rollback + verify] {name}")
    dev, gdn = _dev(), _gdn()
    inp1, inp2 = W.make_inputs(shape, s1), W.make_inputs(shape, s2)
    acc = _accepted(shape, inp1, np.random.default_rng(s2))
    T = shape.n_tok
    # reference path: verify, batched rollback of the entries with a pending rollback, verify
    a = dev.upload(shape, inp1)
    dev.verify(a)
    sel = np.nonzero(acc >= 0)[0]
    if len(sel):
        slots = torch.from_numpy(np.asarray(inp1["slot_ids"], dtype=np.int32)[sel]).cuda()
        gdn.gdn_rollback_batch(a["capture"], slots, torch.from_numpy(acc[sel]).cuda(), len(sel))
    _next_round(a, inp2)
    dev.verify(a)
    # fused path: verify, then verify_resume from the accepted positions
    b = dev.upload(shape, inp1)
    dev.verify(b)
    _next_round(b, inp2)
    dev.verify_resume(b, torch.from_numpy(acc).cuda())
    torch.cuda.synchronize()
    ra, rb = _snapshot(a, T), _snapshot(b, T)
    for k in ra:
        np.testing.assert_array_equal(rb[k], ra[k], err_msg=k)
    say(f"  {W.describe(shape)}: state, conv state, out and capture bit-identical; accepted {acc.tolist()}")


def test_resume_against_oracle_from_the_restored_state():
    """The resumed round equals the oracle's verify of the second round started from the oracle's
    capture at each accepted position of the first (conv window rows bit exact, the rest within
    tolerance)."""
    shape = W.shape_with(W.MULTI_SLOT_VERIFY, n_pool=6, n_batch=5)
    say("[resume vs oracle] 5 slots, 16 tokens, bf16 d=128")
    dev = _dev()
    inp1, inp2 = W.make_inputs(shape, 11), W.make_inputs(shape, 12)
    acc = _accepted(shape, inp1, np.random.default_rng(3))
    o1 = ref.verify_pool(shape, inp1)
    # the second round's starting point per slot: the oracle's capture at the accepted position, or its
    # state after the whole round for entries that start from the slot's state
    inp_r2 = dict(inp1)  # the layer's parameters and slots stay; the activations are the second round's
    for k in ACTS:
        inp_r2[k] = inp2[k]
    st = np.array(inp1["state"], dtype=np.float32, copy=True)
    cs = np.array(inp1["conv_state"], dtype=np.float32, copy=True)
    for b in range(shape.n_batch):
        s = int(inp1["slot_ids"][b])
        if acc[b] >= 0:
            st[s] = o1["cap_ssm"][s, acc[b]]
            cs[s] = o1["cap_conv"][s][acc[b] + 1:acc[b] + 4]
        else:
            st[s] = o1["state"][s]
            cs[s] = o1["conv_state"][s]
    inp_r2["state"], inp_r2["conv_state"] = st, cs
    o2 = ref.verify_pool(shape, inp_r2)
    d = dev.upload(shape, inp1)
    dev.verify(d)
    _next_round(d, inp2)
    dev.verify_resume(d, torch.from_numpy(acc).cuda())
    torch.cuda.synchronize()
    g_st, g_out, g_cap = to_np(d["state"]), to_np(d["out"]), to_np(d["cap_ssm"])
    g_cc, g_cs = to_np(d["cap_conv"]), to_np(d["conv_state"])
    worst = {"state": 0.0, "cap": 0.0, "out": 0.0}
    for b in range(shape.n_batch):
        s = int(inp1["slot_ids"][b])
        np.testing.assert_array_equal(g_cc[s, :3 + shape.n_tok], o2["cap_conv"][s])
        np.testing.assert_array_equal(g_cs[s], o2["conv_state"][s])
        for h in range(shape.n_vh):
            worst["state"] = max(worst["state"], rel_err(g_st[s, h], o2["state"][s, h]))
            worst["out"] = max(worst["out"], out_err(shape, g_out[b, :, h], o2["out"][b, :, h]))
            for t in range(shape.n_tok):
                worst["cap"] = max(worst["cap"], rel_err(g_cap[s, t, h], o2["cap_ssm"][s, t, h]))
    tol = tol_for(shape)
    say(f"  worst rel err {worst} (tol {tol}); accepted {acc.tolist()}")
    for k, v in worst.items():
        assert v <= tol, (k, v, tol)


def test_resume_out_of_range_entry_is_skipped():
    """An entry whose resume position lies outside the capture writes nothing (every launch of a
    multi-launch call skips it); the other entries run normally."""
    shape = W.shape_with(W.SINGLE_SLOT_VERIFY, n_tok=20, n_pool=4, n_batch=3)
    say("[resume out of range] 3 entries, 20 tokens (two launches)")
    dev, gdn = _dev(), _gdn()
    inp1, inp2 = W.make_inputs(shape, 21), W.make_inputs(shape, 22)
    d = dev.upload(shape, inp1)
    dev.verify(d)
    _next_round(d, inp2)
    torch.cuda.synchronize()
    before = _snapshot(d, shape.n_tok)
    d["out"].fill_(7.0)
    bad_b = 1
    acc = np.array([3, shape.n_tok, -1], dtype=np.int32)  # entry 1: position t_cap, outside
    dev.verify_resume(d, torch.from_numpy(acc).cuda())
    torch.cuda.synchronize()
    after = _snapshot(d, shape.n_tok)
    s_bad = int(inp1["slot_ids"][bad_b])
    for k in ("state", "conv_state", "cap_ssm", "cap_conv"):
        np.testing.assert_array_equal(after[k][s_bad], before[k][s_bad], err_msg=k)
    assert np.all(after["out"][bad_b] == 7.0)
    for b in (0, 2):
        assert not np.all(after["out"][b] == 7.0)
        s = int(inp1["slot_ids"][b])
        assert not np.array_equal(after["state"][s], before["state"][s])
    # with GDN_F_CHECK_INDICES the host rejects it before any launch, and nothing changes
    e = dev.upload(shape, inp1, flags=gdn.GDN_F_CHECK_INDICES)
    dev.verify(e)
    torch.cuda.synchronize()
    ref_e = _snapshot(e, shape.n_tok)
    with pytest.raises(gdn.GdnError) as ei:
        dev.verify_resume(e, torch.from_numpy(acc).cuda())
    assert ei.value.code == gdn.GDN_ERR_RANGE
    torch.cuda.synchronize()
    now = _snapshot(e, shape.n_tok)
    for k in ("state", "conv_state", "cap_ssm", "cap_conv"):
        np.testing.assert_array_equal(now[k], ref_e[k], err_msg=k)


DEFER_CASES = {
    "tiny_fp32": (W.shape_with(W.TINY_VERIFY, n_pool=4, n_batch=3), 40, 41, 42),
    "bf16_d128_ten_slots": (W.shape_with(W.MULTI_SLOT_VERIFY, n_pool=12, n_batch=10), 43, 44, 45),
    "bf16_three_launches_37": (W.shape_with(W.SINGLE_SLOT_VERIFY, n_tok=37, n_pool=3, n_batch=2), 46, 47, 48),
}


@pytest.mark.parametrize("name", list(DEFER_CASES))
def test_deferred_commit_leaves_the_state_and_matches_the_commit(name):
    """GDN_F_DEFER_COMMIT: out and capture bit-identical to a committing verify, state and conv
    state untouched; a rollback afterwards gives the committing path's rollback, bit for bit."""
    shape, s1, _, _ = DEFER_CASES[name]
    say(f"[deferred commit] {name}")
    dev, gdn = _dev(), _gdn()
    inp = W.make_inputs(shape, s1)
    acc = _accepted(shape, inp, np.random.default_rng(s1), with_fresh=False)
    a = dev.upload(shape, inp)
    dev.verify(a)
    b = dev.upload(shape, inp, flags=gdn.GDN_F_DEFER_COMMIT)
    dev.verify(b)
    torch.cuda.synchronize()
    ra, rb = _snapshot(a, shape.n_tok), _snapshot(b, shape.n_tok)
    for k in ("out", "cap_ssm", "cap_conv"):
        np.testing.assert_array_equal(rb[k], ra[k], err_msg=k)
    np.testing.assert_array_equal(rb["state"], np.asarray(inp["state"], dtype=np.float32))
    np.testing.assert_array_equal(rb["conv_state"], np.asarray(inp["conv_state"], dtype=np.float32))
    slots = torch.from_numpy(np.asarray(inp["slot_ids"], dtype=np.int32)).cuda()
    acc_t = torch.from_numpy(acc).cuda()
    for d in (a, b):
        gdn.gdn_rollback_batch(d["capture"], slots, acc_t, shape.n_batch)
    torch.cuda.synchronize()
    ra, rb = _snapshot(a, shape.n_tok), _snapshot(b, shape.n_tok)
    for k in ("state", "conv_state"):
        np.testing.assert_array_equal(rb[k], ra[k], err_msg=k)


@pytest.mark.parametrize("name", list(DEFER_CASES))
def test_deferred_commit_then_trim_equals_the_committing_path(name):
    """The trim form after a verify whose commit was deferred: trim 0 commits the last position (the
    committing verify's own final state), trim > 0 restores position n_tok - 1 - trim; both bit for
    bit what the committing verify followed by the same trim leaves."""
    shape, s1, _, _ = DEFER_CASES[name]
    say(f"[deferred commit + trim] {name}")
    dev, gdn = _dev(), _gdn()
    inp = W.make_inputs(shape, s1 + 100)
    trims = [0] + [int(t) for t in np.asarray(inp["trims"])[1:]]
    a = dev.upload(shape, inp)
    b = dev.upload(shape, inp, flags=gdn.GDN_F_DEFER_COMMIT)
    dev.verify(a)
    dev.verify(b)
    for b_ in range(shape.n_batch):
        s = int(inp["slot_ids"][b_])
        for d in (a, b):
            gdn.gdn_rollback_trim(d["capture"], s, trims[b_], shape.n_tok)
    torch.cuda.synchronize()
    ra, rb = _snapshot(a, shape.n_tok), _snapshot(b, shape.n_tok)
    for k in ("state", "conv_state"):
        np.testing.assert_array_equal(rb[k], ra[k], err_msg=k)
    # the slot with trim 0 holds the state after every token, as the committing verify left it
    s0 = int(inp["slot_ids"][0])
    np.testing.assert_array_equal(rb["state"][s0], ra["cap_ssm"][s0, shape.n_tok - 1])
    say(f"  {W.describe(shape)}: trims {trims} bit-identical")


@pytest.mark.parametrize("name", list(DEFER_CASES))
def test_deferred_resume_rounds_equal_committed_rounds(name):
    """Three rounds of the resume protocol with the commit deferred (verify, then verify_resume
    from each accepted position, a final rollback to materialise the state) against three rounds
    of verify + rollback: every output, the last capture and the committed state bit-identical."""
    shape, s1, s2, s3 = DEFER_CASES[name]
    say(f"[deferred resume rounds] {name}")
    dev, gdn = _dev(), _gdn()
    rounds = [W.make_inputs(shape, s) for s in (s1, s2, s3)]
    accs = [_accepted(shape, r, np.random.default_rng(7 + i), with_fresh=False) for i, r in enumerate(rounds)]
    slots = torch.from_numpy(np.asarray(rounds[0]["slot_ids"], dtype=np.int32)).cuda()
    a = dev.upload(shape, rounds[0])
    b = dev.upload(shape, rounds[0], flags=gdn.GDN_F_DEFER_COMMIT)
    outs_a, outs_b = [], []
    for i, inp in enumerate(rounds):
        acc_t = torch.from_numpy(accs[i]).cuda()
        if i > 0:
            _next_round(a, inp)
            _next_round(b, inp)
        dev.verify(a)
        gdn.gdn_rollback_batch(a["capture"], slots, acc_t, shape.n_batch)
        if i == 0:
            dev.verify(b)
        else:
            dev.verify_resume(b, torch.from_numpy(accs[i - 1]).cuda())
        torch.cuda.synchronize()
        outs_a.append(to_np(a["out"].float()))
        outs_b.append(to_np(b["out"].float()))
    gdn.gdn_rollback_batch(b["capture"], slots, torch.from_numpy(accs[-1]).cuda(), shape.n_batch)
    torch.cuda.synchronize()
    for i in range(len(rounds)):
        np.testing.assert_array_equal(outs_b[i], outs_a[i], err_msg=f"out of round {i}")
    ra, rb = _snapshot(a, shape.n_tok), _snapshot(b, shape.n_tok)
    for k in ("state", "conv_state", "cap_ssm", "cap_conv"):
        np.testing.assert_array_equal(rb[k], ra[k], err_msg=k)
    say(f"  {W.describe(shape)}: three rounds bit-identical")


def _slice(inp: dict, n: int) -> dict:
    """The first n batch entries of a call's inputs (the pool, parameters and slots stay)."""
    out = dict(inp)
    for k in ("qkv", "z", "alpha", "beta", "slot_ids", "trims"):
        out[k] = np.asarray(inp[k])[:n]
    return out


@pytest.mark.parametrize("name,shape,n_big", [
    ("one_slot_16", W.shape_with(W.SINGLE_SLOT_VERIFY, n_pool=6, n_batch=1), 5),
    ("two_slots_gqa4_37", W.shape_with(W.SINGLE_SLOT_VERIFY, n_kh=4, n_vh=16, n_tok=37, n_pool=18, n_batch=2), 17),
    ("one_slot_qk_norm_5", W.shape_with(W.SINGLE_SLOT_VERIFY, n_tok=5, n_pool=6, n_batch=1), 5),
])
def test_workgroup_per_value_head_equals_per_key_head(name, shape, n_big):
    """With few batch entries gdn_verify runs a workgroup per value head (8 waves); the same entries
    inside a call of n_big entries (more than 64 workgroups per key head) run a workgroup per key
    head.  Out, state, conv state and capture of the shared entries agree bit for bit, plain and
    resuming from accepted positions with the commit deferred."""
    say(f"[value-head vs key-head workgroups] {name}")
    dev, gdn = _dev(), _gdn()
    flags = gdn.GDN_F_QK_NORM_SILU if "qk_norm" in name else 0
    big = W.shape_with(shape, n_batch=n_big)
    inp_big = W.make_inputs(big, 61)
    inp = _slice(inp_big, shape.n_batch)
    n, T = shape.n_batch, shape.n_tok
    for defer in (False, True):
        fl = flags | (gdn.GDN_F_DEFER_COMMIT if defer else 0)
        a = dev.upload(shape, inp, flags=fl)
        b = dev.upload(big, inp_big, flags=fl)
        dev.verify(a)
        dev.verify(b)
        if defer:  # a second round resuming from each entry's last position
            acc = np.full(n, T - 1, dtype=np.int32)
            dev.verify_resume(a, torch.from_numpy(acc).cuda())
            dev.verify_resume(b, torch.from_numpy(np.full(n_big, T - 1, dtype=np.int32)).cuda())
        torch.cuda.synchronize()
        ra, rb = _snapshot(a, T), _snapshot(b, T)
        np.testing.assert_array_equal(ra["out"], rb["out"][:n], err_msg="out")
        for k in ("state", "conv_state", "cap_ssm", "cap_conv"):
            for e in range(n):
                sl = int(inp["slot_ids"][e])
                np.testing.assert_array_equal(ra[k][sl], rb[k][sl], err_msg=f"{k} defer={defer}")
