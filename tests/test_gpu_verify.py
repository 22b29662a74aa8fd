"""GPU parity of chain verify and rollback against the fp64 oracle (through the C ABI)."""

import numpy as np
import pytest

from gated_deltanet_linear_verify_amd import workloads as W
from oracle import ref
from tests.gpu_util import out_err, out_err_slices, rel_err, rel_err_slices, say, to_np, tol_for

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


def _check_pool(shape, inp, d, tol, *, flags=0, check_capture=True):
    """Compare every output of a small verify call with the oracle."""
    o = ref.verify_pool(shape, inp, flags=flags)
    st = to_np(d["state"])
    out = to_np(d["out"])
    worst = {"state": 0.0, "cap": 0.0, "out": 0.0}
    for b in range(shape.n_batch):
        s = int(inp["slot_ids"][b])
        for h in range(shape.n_vh):
            worst["state"] = max(worst["state"], rel_err(st[s, h], o["state"][s, h]))
            worst["out"] = max(worst["out"], out_err(shape, out[b, :, h], o["out"][b, :, h]))
    if check_capture:
        cap = to_np(d["cap_ssm"])
        for b in range(shape.n_batch):
            s = int(inp["slot_ids"][b])
            for h in range(shape.n_vh):
                for t in range(shape.n_tok):
                    worst["cap"] = max(worst["cap"], rel_err(cap[s, t, h], o["cap_ssm"][s, t, h]))
        # conv window and conv state are copies: bit exact
        cc = to_np(d["cap_conv"])
        for b in range(shape.n_batch):
            s = int(inp["slot_ids"][b])
            np.testing.assert_array_equal(cc[s, :3 + shape.n_tok], o["cap_conv"][s])
    np.testing.assert_array_equal(to_np(d["conv_state"]), o["conv_state"])
    # slots not in the batch are untouched, bit for bit
    used = set(int(x) for x in inp["slot_ids"])
    for s in range(shape.n_pool):
        if s not in used:
            np.testing.assert_array_equal(st[s], inp["state"][s])
    say(f"  {W.describe(shape)} worst rel err {worst} (tol {tol})")
    for k, v in worst.items():
        assert v <= tol, (k, v, tol)
    return o


CASES = {
    # name: (shape, flags)
    "tiny_verify": (W.TINY_VERIFY, 0),
    "single_slot_verify": (W.SINGLE_SLOT_VERIFY, 0),
    "ragged_three_tiles": (W.shape_with(W.SINGLE_SLOT_VERIFY, n_tok=37, n_pool=3, n_batch=2), 0),
    "one_token": (W.shape_with(W.SINGLE_SLOT_VERIFY, n_tok=1, n_pool=2, n_batch=2), 0),
    # one value head per workgroup, and a second launch of one token: the key heads' q / k conv
    # state is rebuilt from the old rows after it
    "split_tail_of_one_token": (W.shape_with(W.SINGLE_SLOT_VERIFY, n_tok=17, n_pool=2, n_batch=1), 0),
    "split_gqa4_tail_of_two": (W.shape_with(W.SINGLE_SLOT_VERIFY, n_kh=4, n_vh=16, n_tok=18, n_pool=3,
                                            n_batch=2), 0),
    "two_tokens_conv_from_state": (W.shape_with(W.TINY_VERIFY, n_tok=2, n_pool=4, n_batch=3), 0),
    "fp32_act_bf16_out": (W.shape_with(W.TINY_VERIFY, out_dtype=W.BF16, n_tok=17), 0),
    "bf16_act_fp32_out": (W.shape_with(W.SINGLE_SLOT_VERIFY, out_dtype=W.F32, n_vh=16, n_kh=16), 0),
    "gqa4_d128": (W.shape_with(W.SINGLE_SLOT_VERIFY, n_kh=4, n_vh=16, n_tok=9), 0),
    "gqa8_d64": (W.shape_with(W.TINY_VERIFY, n_kh=1, n_vh=8, n_tok=5), 0),
    "qk_norm_silu_flag": (W.shape_with(W.SINGLE_SLOT_VERIFY, n_tok=12), 1),
    "qk_norm_silu_fp32": (W.shape_with(W.TINY_VERIFY, n_tok=20), 1),
}


@pytest.mark.parametrize("name", list(CASES))
def test_verify_parity(name):
    shape, flags = CASES[name]
    say(f"[verify parity] {name}")
    inp = W.make_inputs(shape, 0)
    dev = _dev()
    gdn = _gdn()
    d = dev.upload(shape, inp, flags=(gdn.GDN_F_QK_NORM_SILU if flags else 0))
    dev.verify(d)
    torch.cuda.synchronize()
    _check_pool(shape, inp, d, tol_for(shape), flags=flags)


def test_verify_without_capture_matches_capture_path():
    shape = W.shape_with(W.SINGLE_SLOT_VERIFY, n_pool=2, n_batch=2, n_tok=7)
    inp = W.make_inputs(shape, 3)
    dev = _dev()
    a = dev.upload(shape, inp)
    b = dev.upload(shape, inp, capture=False)
    dev.verify(a)
    dev.verify(b, with_capture=False)
    torch.cuda.synchronize()
    assert torch.equal(a["state"], b["state"])
    assert torch.equal(a["conv_state"], b["conv_state"])
    assert torch.equal(a["out"], b["out"])


@pytest.mark.parametrize("where", ["fresh_stream", "stream_with_scratch"])
def test_single_slot_verify_captured_in_a_graph_matches_eager(where):
    """One slot x 16 tokens (the launch that splits each head's rows over four workgroups and
    normalises in a second kernel) recorded under torch's stream capture and replayed three times,
    the committed state restored in between with eager work and a synchronisation: every replay
    leaves the eager call's state, conv state, captures and outputs bit for bit.  Captured on a
    fresh stream the call must not allocate a readout scratch, and captured on a stream whose eager
    launch already holds one it must not record that buffer (a replay on another stream could run
    alongside that stream's later calls): both record the one-kernel path."""
    shape = W.SINGLE_SLOT_VERIFY
    say(f"[verify graph] 1 slot x 16, {where}")
    inp = W.make_inputs(shape, 31)
    dev = _dev()
    d = dev.upload(shape, inp, fill_capture=0.0)
    st0, cs0 = d["state"].clone(), d["conv_state"].clone()
    keys = ("out", "state", "conv_state", "cap_ssm", "cap_conv")
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        dev.verify(d)
    torch.cuda.synchronize()
    want = {k: d[k].clone() for k in keys}
    _check_pool(shape, inp, d, tol_for(shape))
    g = torch.cuda.CUDAGraph()
    d["state"].copy_(st0)
    d["conv_state"].copy_(cs0)
    torch.cuda.synchronize()
    if where == "fresh_stream":
        with torch.cuda.graph(g, stream=torch.cuda.Stream()):
            dev.verify(d)
    else:
        with torch.cuda.graph(g, stream=side):
            dev.verify(d)
    for rep in range(3):
        d["state"].copy_(st0)
        d["conv_state"].copy_(cs0)
        d["out"].fill_(7.0)
        d["cap_ssm"].fill_(7.0)
        with torch.cuda.stream(side):  # eager work on the capture's stream between replays
            dev.verify(dev.upload(shape, W.make_inputs(shape, 40 + rep)))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in keys:
            assert torch.equal(d[k], want[k]), (rep, k)


def test_verify_is_deterministic():
    shape = W.shape_with(W.MULTI_SLOT_VERIFY, n_pool=8, n_batch=8)
    inp = W.make_inputs(shape, 4)
    dev = _dev()
    a = dev.upload(shape, inp)
    b = dev.upload(shape, inp)
    dev.verify(a)
    dev.verify(b)
    torch.cuda.synchronize()
    for k in ("state", "conv_state", "out", "cap_ssm", "cap_conv"):
        assert torch.equal(a[k], b[k]), k


@pytest.mark.parametrize("n_batch", [2, 3, 8])
def test_slot_permutation_gives_the_same_per_slot_results(n_batch):
    """Batch entries listed in reverse order (their inputs and slot ids permuted together) leave
    every slot with the same state, conv state and capture, bit for bit, and each entry's output
    moves with it.  2 entries take the row split, 3 a workgroup per value head, 8 a workgroup per
    key head."""
    shape = W.shape_with(W.SINGLE_SLOT_VERIFY, n_pool=n_batch + 2, n_batch=n_batch)
    say(f"[slot permutation] {n_batch} entries")
    inp = W.make_inputs(shape, 11)
    perm = np.arange(n_batch)[::-1].copy()
    pinp = dict(inp)
    for k in ("qkv", "z", "alpha", "beta", "slot_ids"):
        pinp[k] = np.ascontiguousarray(np.asarray(inp[k])[perm])
    dev = _dev()
    a = dev.upload(shape, inp, fill_capture=0.0)  # the pool's unused slots keep a comparable fill
    b = dev.upload(shape, pinp, fill_capture=0.0)
    dev.verify(a)
    dev.verify(b)
    torch.cuda.synchronize()
    for k in ("state", "conv_state", "cap_ssm", "cap_conv"):
        assert torch.equal(a[k], b[k]), k
    assert torch.equal(a["out"][torch.from_numpy(perm).cuda()], b["out"])


@pytest.mark.parametrize("base", ["single_slot", "tiny_fp32"])
def test_extreme_gates_and_gate_inputs(base):
    """alpha far into both tails of softplus (rho down to e^-82, or 1 to the last bit), beta at 0
    and 1, and z far into both tails of the SiLU, against the oracle at the usual bar.  Larger
    alpha is left out: there rho, and with beta = 0 the whole state, falls below fp32's normal range
    (2^-126), which an fp32 state cannot hold, so a relative comparison with the fp64 oracle has no
    meaning."""
    shape = W.shape_with(W.SINGLE_SLOT_VERIFY if base == "single_slot" else W.TINY_VERIFY, n_tok=16)
    say(f"[extreme gates] {base}")
    inp = W.make_inputs(shape, 12)
    T, H = shape.n_tok, shape.n_vh
    alpha = np.asarray(inp["alpha"]).copy()
    beta = np.asarray(inp["beta"]).copy()
    z = np.asarray(inp["z"]).copy()
    for t in range(T):
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
    dev = _dev()
    d = dev.upload(shape, inp)
    dev.verify(d)
    torch.cuda.synchronize()
    _check_pool(shape, inp, d, tol_for(shape))


def test_beta_zero_no_decay_is_identity_on_gpu():
    shape = W.shape_with(W.SINGLE_SLOT_VERIFY, n_tok=5)
    inp = W.make_inputs(shape, 5)
    inp["beta"][:] = 0.0
    inp["alpha"][:] = -1e30
    dev = _dev()
    d = dev.upload(shape, inp)
    dev.verify(d)
    torch.cuda.synchronize()
    st = to_np(d["state"])
    np.testing.assert_array_equal(st, inp["state"])
    cap = to_np(d["cap_ssm"])
    for t in range(shape.n_tok):
        np.testing.assert_array_equal(cap[:, t], inp["state"])


@pytest.mark.parametrize("shape_name", ["tiny_verify", "single_slot_verify"])
def test_rollback_equals_shorter_verify(shape_name):
    """verify(T) + rollback(a) leaves bit for bit what verify(a+1) leaves, for every a; and
    both match the oracle's state after a+1 tokens."""
    base = W.WORKLOADS[shape_name]
    shape = W.shape_with(base, n_pool=3, n_batch=2)
    inp = W.make_inputs(shape, 6)
    dev = _dev()
    gdn = _gdn()
    full = dev.upload(shape, inp)
    dev.verify(full)
    torch.cuda.synchronize()
    cap_ssm = full["cap_ssm"].clone()
    cap_conv = full["cap_conv"].clone()
    tol = tol_for(shape)
    for a in range(shape.n_tok):
        say(f"[rollback] {shape_name} a={a}")
        short_shape = W.shape_with(shape, n_tok=a + 1)
        sinp = dict(inp)
        for k in ("qkv", "z", "alpha", "beta"):
            sinp[k] = np.ascontiguousarray(inp[k][:, :a + 1])
        short = dev.upload(short_shape, sinp)
        dev.verify(short)
        # restore into a fresh copy of the full call's capture
        rb = dev.upload(shape, inp)
        rb["cap_ssm"].copy_(cap_ssm)
        rb["cap_conv"].copy_(cap_conv)
        for b in range(shape.n_batch):
            gdn.gdn_rollback(rb["capture"], int(inp["slot_ids"][b]), a)
        torch.cuda.synchronize()
        assert torch.equal(rb["state"], short["state"])
        assert torch.equal(rb["conv_state"], short["conv_state"])
        o = ref.verify_pool(short_shape, sinp)
        st = to_np(rb["state"])
        for b in range(shape.n_batch):
            s = int(inp["slot_ids"][b])
            for h in range(shape.n_vh):
                assert rel_err(st[s, h], o["state"][s, h]) <= tol


def test_rollback_batch_and_trim_multi_slot():
    """Per-slot random trims through the batched rollback == per-slot single rollbacks == the
    capture element accepted_idx = K - trim, bit for bit."""
    shape = W.shape_with(W.MULTI_SLOT_VERIFY, n_pool=12, n_batch=10)
    inp = W.make_inputs(shape, 7)
    dev = _dev()
    gdn = _gdn()
    d = dev.upload(shape, inp)
    dev.verify(d)
    torch.cuda.synchronize()
    K = shape.n_tok - 1
    trims = inp["trims"]
    acc = np.array([K - int(t) for t in trims], dtype=np.int32)
    cap_ssm = to_np(d["cap_ssm"])
    cap_conv = to_np(d["cap_conv"])
    state_after_verify = to_np(d["state"])
    slots_t = d["slot_ids"]
    acc_t = torch.from_numpy(acc).cuda()
    gdn.gdn_rollback_batch(d["capture"], slots_t, acc_t, shape.n_batch)
    torch.cuda.synchronize()
    st = to_np(d["state"])
    cs = to_np(d["conv_state"])
    for b in range(shape.n_batch):
        s = int(inp["slot_ids"][b])
        np.testing.assert_array_equal(st[s], cap_ssm[s, acc[b]])
        np.testing.assert_array_equal(cs[s], cap_conv[s, acc[b] + 1:acc[b] + 4])
    # trim form on a second copy: trim 0 is a no-op, otherwise the same restore
    e = dev.upload(shape, inp)
    dev.verify(e)
    for b in range(shape.n_batch):
        gdn.gdn_rollback_trim(e["capture"], int(inp["slot_ids"][b]), int(trims[b]), shape.n_tok)
    torch.cuda.synchronize()
    st2 = to_np(e["state"])
    for b in range(shape.n_batch):
        s = int(inp["slot_ids"][b])
        if trims[b] == 0:
            np.testing.assert_array_equal(st2[s], state_after_verify[s])
        np.testing.assert_array_equal(st2[s], st[s])
    with pytest.raises(gdn.GdnError) as ei:
        gdn.gdn_rollback_trim(e["capture"], 0, shape.n_tok, shape.n_tok)
    assert ei.value.code == gdn.GDN_ERR_RANGE


def test_multi_slot_full_size_every_unit():
    """The 64-slot workload at full size, in the benchmark's launch configuration: every (slot,
    head) unit's final state, every output and every capture position against the oracle (the
    oracle runs eight slots at a time to bound host memory), the conv window and conv state bit
    exact for every slot."""
    shape = W.MULTI_SLOT_VERIFY
    inp = W.make_inputs(shape, 0)
    dev = _dev()
    d = dev.upload(shape, inp)
    dev.verify(d)
    torch.cuda.synchronize()
    st = to_np(d["state"])
    out = to_np(d["out"])
    tol = tol_for(shape)
    worst = {"state": 0.0, "out": 0.0, "cap": 0.0}
    group = 8
    for b0 in range(0, shape.n_batch, group):
        bs = np.arange(b0, min(b0 + group, shape.n_batch))
        ub = np.repeat(bs, shape.n_vh).astype(np.int32)
        uh = np.tile(np.arange(shape.n_vh), len(bs)).astype(np.int32)
        o = ref.verify_units(shape, inp, (ub, uh))
        slots = np.asarray(inp["slot_ids"])[ub]
        worst["state"] = max(worst["state"], float(rel_err_slices(st[slots, uh], o["state"], 1).max()))
        worst["out"] = max(worst["out"], float(out_err_slices(shape, out[ub, :, uh], o["y"], 1).max()))
        cap = to_np(d["cap_ssm"][torch.from_numpy(np.asarray(inp["slot_ids"])[bs]).long().cuda()])
        cap = cap.transpose(0, 2, 1, 3, 4).reshape(len(ub), shape.n_tok, shape.d_v, shape.d_k)
        worst["cap"] = max(worst["cap"], float(rel_err_slices(cap, o["cap"], 2).max()))
        del o, cap
    say(f"  multi-slot, all {shape.n_batch * shape.n_vh} units: worst rel err {worst} (tol {tol})")
    for k, v in worst.items():
        assert v <= tol, (k, v, tol)
    win = ref.conv_window(shape, inp)
    cc = to_np(d["cap_conv"])
    cs = to_np(d["conv_state"])
    for b in range(shape.n_batch):
        s = int(inp["slot_ids"][b])
        np.testing.assert_array_equal(cc[s], win[b])
        np.testing.assert_array_equal(cs[s], win[b, -3:])


def test_check_indices_rejects_bad_slots_without_mutation():
    gdn = _gdn()
    dev = _dev()
    shape = W.shape_with(W.TINY_VERIFY, n_pool=4, n_batch=2)
    inp = W.make_inputs(shape, 8)
    for bad in ([1, 1], [0, 4], [-1, 2]):
        inp2 = dict(inp)
        inp2["slot_ids"] = np.array(bad, dtype=np.int32)
        d = dev.upload(shape, inp2, flags=gdn.GDN_F_CHECK_INDICES)
        before = d["state"].clone()
        with pytest.raises(gdn.GdnError) as ei:
            dev.verify(d)
        assert ei.value.code == gdn.GDN_ERR_RANGE
        torch.cuda.synchronize()
        assert torch.equal(before, d["state"])


def test_check_indices_under_capture_is_refused_and_the_capture_survives():
    """With GDN_F_CHECK_INDICES a call on a capturing stream returns GDN_ERR_ARG before touching
    the stream (its host copy cannot be recorded); the capture goes on, and a verify recorded after
    it replays to the eager call's results bit for bit."""
    gdn = _gdn()
    dev = _dev()
    shape = W.shape_with(W.TINY_VERIFY, n_pool=3, n_batch=2, n_tok=5)
    inp = W.make_inputs(shape, 18)
    checked = dev.upload(shape, inp, flags=gdn.GDN_F_CHECK_INDICES)
    eager = dev.upload(shape, inp, fill_capture=0.0)
    graph = dev.upload(shape, inp, fill_capture=0.0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        with pytest.raises(gdn.GdnError) as ei:
            dev.verify(checked)
        dev.verify(graph)
    assert ei.value.code == gdn.GDN_ERR_ARG
    dev.verify(eager)
    g.replay()
    torch.cuda.synchronize()
    for k in ("out", "state", "conv_state", "cap_ssm", "cap_conv"):
        assert torch.equal(eager[k], graph[k]), k


def test_out_of_range_slot_is_skipped_by_the_kernel():
    """Without the host check, an entry whose slot is outside the pool is skipped (its bounds
    check in the kernel stops it before any access); the other entries are unaffected."""
    dev = _dev()
    shape = W.shape_with(W.TINY_VERIFY, n_pool=3, n_batch=2)
    inp = W.make_inputs(shape, 9)
    good = dev.upload(shape, inp)
    dev.verify(good)
    inp2 = dict(inp)
    inp2["slot_ids"] = np.array([int(inp["slot_ids"][0]), 7], dtype=np.int32)
    d = dev.upload(shape, inp2)
    dev.verify(d)
    torch.cuda.synchronize()
    s0 = int(inp["slot_ids"][0])
    assert torch.equal(d["state"][s0], good["state"][s0])
    others = [s for s in range(3) if s != s0]
    for s in others:
        np.testing.assert_array_equal(to_np(d["state"][s]), inp["state"][s])


def test_reset_zeroes_one_slot():
    gdn = _gdn()
    dev = _dev()
    shape = W.shape_with(W.TINY_VERIFY, n_pool=3)
    inp = W.make_inputs(shape, 10)
    d = dev.upload(shape, inp)
    gdn.gdn_reset(d["dims"], d["state"], d["conv_state"], 1)
    torch.cuda.synchronize()
    st = to_np(d["state"])
    assert np.all(st[1] == 0) and np.all(to_np(d["conv_state"])[1] == 0)
    np.testing.assert_array_equal(st[0], inp["state"][0])
    np.testing.assert_array_equal(st[2], inp["state"][2])
