"""GPU parity of tree verify (and tree-mode rollback) against the fp64 oracle, through the C ABI."""

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
    gdn.lib()


def _mods():
    from gated_deltanet_linear_verify_amd import device, gdn
    return device, gdn


def _tree_upload(shape, inp, **kw):
    device, gdn = _mods()
    return device.upload(shape, inp, mode=gdn.GDN_TREE, **kw)


def _check_tree(shape, inp, d, units=None, flags=0, out_tol=None):
    """Node states, node outputs and per-node conv states against the oracle.  out_tol, if given,
    maps the oracle's result to per-(unit, node) output tolerances [U][T]."""
    o = ref.tree_units(shape, inp, units, flags=flags)
    tol = tol_for(shape)
    otol = np.full((len(o["units"][0]), shape.n_tok), tol) if out_tol is None else out_tol(o)
    cap = d["cap_ssm"]
    out = to_np(d["out"])
    worst_s, worst_o = 0.0, 0.0
    ub, uh = o["units"]
    for u in range(len(ub)):
        b, h = int(ub[u]), int(uh[u])
        s = int(inp["slot_ids"][b])
        c = to_np(cap[s, :, h])
        for i in range(shape.n_tok):
            worst_s = max(worst_s, rel_err(c[i], o["cap"][u, i]))
            worst_o = max(worst_o, out_err(shape, out[b, i, h], o["y"][u, i]) / otol[u, i] * tol)
    cc = to_np(d["cap_conv"])
    expect_cc = ref.tree_conv(shape, inp)
    for b in range(shape.n_batch):
        s = int(inp["slot_ids"][b])
        np.testing.assert_array_equal(cc[s, :shape.n_tok], expect_cc[b])
    say(f"  tree {W.describe(shape)} worst rel err state {worst_s:.2e} out {worst_o:.2e}"
        + ("" if out_tol is None else " (out scaled to the per-node bar)"))
    assert worst_s <= tol and worst_o <= tol


TREE_CASES = {
    "tiny_fp32_depth3": (W.shape_with(W.TINY_VERIFY, n_tok=12, n_pool=2, n_batch=2), 3, 0),
    "bf16_d128_depth8": (W.shape_with(W.TREE_VERIFY, n_pool=3, n_batch=2, n_tok=40), 8, 0),
    "bf16_d128_64_nodes": (W.shape_with(W.TREE_VERIFY, n_pool=2, n_batch=1), 8, 0),
    "deep_comb": (W.shape_with(W.TINY_VERIFY, n_tok=30, act_dtype=W.BF16, out_dtype=W.BF16), 64, 0),
    "qk_norm_flag": (W.shape_with(W.TREE_VERIFY, n_pool=1, n_batch=1, n_tok=20), 5, 1),
    # more nodes than one launch holds (64): consecutive launches, nodes whose parent is in an
    # earlier launch start from its capture, conv windows reach back into earlier launches
    "bf16_d128_root_plus_64": (W.shape_with(W.TREE_VERIFY, n_pool=2, n_batch=2, n_tok=65), 8, 0),
    "bf16_d128_128_nodes": (W.shape_with(W.TREE_VERIFY, n_pool=2, n_batch=2, n_tok=128), 8, 0),
    "fp32_d64_200_nodes_depth12": (W.shape_with(W.TINY_VERIFY, n_tok=200, n_pool=2, n_batch=2), 12, 0),
    "bf16_d64_deep_comb_150": (W.shape_with(W.TINY_VERIFY, n_tok=150, act_dtype=W.BF16, out_dtype=W.BF16), 150, 0),
    # the most nodes one call takes: 16 consecutive launches of 64
    "fp32_d64_1024_nodes_max": (W.shape_with(W.TINY_VERIFY, n_tok=1024, n_pool=1, n_batch=1), 16, 0),
}


@pytest.mark.parametrize("name", list(TREE_CASES))
def test_tree_parity(name):
    shape, depth, flags = TREE_CASES[name]
    say(f"[tree parity] {name}")
    device, gdn = _mods()
    inp = W.make_tree_inputs(shape, 0)
    rng = np.random.default_rng(5)
    inp["parent"] = np.stack([W.random_tree(rng, shape.n_tok, depth) for _ in range(shape.n_batch)])
    d = _tree_upload(shape, inp, flags=(gdn.GDN_F_QK_NORM_SILU if flags else 0))
    st0 = d["state"].clone()
    cs0 = d["conv_state"].clone()
    device.verify_tree(d)
    torch.cuda.synchronize()
    # tree verify leaves the committed state alone
    assert torch.equal(d["state"], st0) and torch.equal(d["conv_state"], cs0)
    _check_tree(shape, inp, d, flags=flags)


def test_tree_full_size_every_unit():
    """The 8-slot, 64-node tree workload at full size: every (slot, head) unit's node states and
    node outputs against the oracle (two slots at a time, to bound host memory), per-node conv
    states bit exact."""
    shape = W.TREE_VERIFY
    device, gdn = _mods()
    inp = W.make_tree_inputs(shape, 0)
    d = _tree_upload(shape, inp)
    device.verify_tree(d)
    torch.cuda.synchronize()
    out = to_np(d["out"])
    worst_s, worst_o = 0.0, 0.0
    for b0 in range(0, shape.n_batch, 2):
        bs = np.arange(b0, min(b0 + 2, shape.n_batch))
        ub = np.repeat(bs, shape.n_vh).astype(np.int32)
        uh = np.tile(np.arange(shape.n_vh), len(bs)).astype(np.int32)
        o = ref.tree_units(shape, inp, (ub, uh))
        cap = to_np(d["cap_ssm"][torch.from_numpy(np.asarray(inp["slot_ids"])[bs]).long().cuda()])
        cap = cap.transpose(0, 2, 1, 3, 4).reshape(len(ub), shape.n_tok, shape.d_v, shape.d_k)
        worst_s = max(worst_s, float(rel_err_slices(cap, o["cap"], 2).max()))
        worst_o = max(worst_o, float(out_err_slices(shape, out[ub, :, uh][:, :, None, :],
                                                    o["y"][:, :, None, :], 2).max()))
        del o, cap
    cc = to_np(d["cap_conv"])
    expect_cc = ref.tree_conv(shape, inp)
    for b in range(shape.n_batch):
        s = int(inp["slot_ids"][b])
        np.testing.assert_array_equal(cc[s, :shape.n_tok], expect_cc[b])
    say(f"  tree, all {shape.n_batch * shape.n_vh} units: worst rel err state {worst_s:.2e} out {worst_o:.2e}")
    tol = tol_for(shape)
    assert worst_s <= tol and worst_o <= tol


@pytest.mark.parametrize("n_tok", [16, 100])
def test_chain_shaped_tree_equals_chain_verify_bitwise(n_tok):
    """A chain-shaped tree gives the chain verify's captures and outputs bit for bit; at 100 nodes
    the tree runs as two launches and the chain as seven, each carrying its state over."""
    shape = W.shape_with(W.SINGLE_SLOT_VERIFY, n_pool=2, n_batch=2, n_tok=n_tok)
    device, gdn = _mods()
    inp = W.make_inputs(shape, 3)
    inp["parent"] = np.stack([W.chain_parents(shape.n_tok)] * shape.n_batch)
    t = _tree_upload(shape, inp)
    device.verify_tree(t)
    c = device.upload(shape, inp)
    device.verify(c)
    torch.cuda.synchronize()
    for b in range(shape.n_batch):
        s = int(inp["slot_ids"][b])
        assert torch.equal(t["cap_ssm"][s], c["cap_ssm"][s])
    assert torch.equal(t["out"], c["out"])
    # per-node conv state of a chain = rows i+1 .. i+3 of the chain's conv window
    for b in range(shape.n_batch):
        s = int(inp["slot_ids"][b])
        for i in range(shape.n_tok):
            assert torch.equal(t["cap_conv"][s, i], c["cap_conv"][s, i + 1:i + 4])


@pytest.mark.parametrize("n_tok", [48, 130])
def test_tree_rollback_equals_chain_along_accepted_path(n_tok):
    """Commit an accepted node with gdn_rollback (tree mode): state and conv state equal a chain
    verify of the node's root path, bit for bit (at 130 nodes, three launches)."""
    shape = W.shape_with(W.TREE_VERIFY, n_pool=3, n_batch=2, n_tok=n_tok)
    device, gdn = _mods()
    inp = W.make_tree_inputs(shape, 7)
    t = _tree_upload(shape, inp)
    device.verify_tree(t)
    torch.cuda.synchronize()
    for b in range(shape.n_batch):
        s = int(inp["slot_ids"][b])
        a = int(inp["accepted"][b])
        gdn.gdn_rollback(t["capture"], s, a)
        path = []
        n = a
        while n >= 0:
            path.append(n)
            n = int(inp["parent"][b, n])
        path.reverse()
        say(f"  slot {s} accepted node {a}, path length {len(path)}")
        sub = W.shape_with(shape, n_tok=len(path), n_batch=1)
        sinp = dict(inp)
        for k in ("qkv", "z", "alpha", "beta"):
            sinp[k] = np.ascontiguousarray(inp[k][b:b + 1, path])
        sinp["slot_ids"] = inp["slot_ids"][b:b + 1]
        c = device.upload(sub, sinp)
        device.verify(c)
        torch.cuda.synchronize()
        assert torch.equal(t["state"][s], c["state"][s])
        assert torch.equal(t["conv_state"][s], c["conv_state"][s])


def test_tree_slot_permutation_gives_the_same_per_slot_results():
    """Tree entries listed in reverse order (inputs, parent arrays and slot ids permuted together)
    give every slot the same node captures bit for bit, and each entry's outputs move with it; the
    committed state is untouched either way."""
    device, gdn = _mods()
    shape = W.shape_with(W.TREE_VERIFY, n_pool=5, n_batch=3, n_tok=40)
    say("[tree slot permutation] 3 entries x 40 nodes")
    inp = W.make_tree_inputs(shape, 2)
    rng = np.random.default_rng(8)
    inp["parent"] = np.stack([W.random_tree(rng, shape.n_tok, 8) for _ in range(shape.n_batch)])
    perm = np.arange(shape.n_batch)[::-1].copy()
    pinp = dict(inp)
    for k in ("qkv", "z", "alpha", "beta", "slot_ids", "parent"):
        pinp[k] = np.ascontiguousarray(np.asarray(inp[k])[perm])
    a = _tree_upload(shape, inp, fill_capture=0.0)
    b = _tree_upload(shape, pinp, fill_capture=0.0)
    device.verify_tree(a)
    device.verify_tree(b)
    torch.cuda.synchronize()
    for k in ("state", "conv_state", "cap_ssm", "cap_conv"):
        assert torch.equal(a[k], b[k]), k
    assert torch.equal(a["out"][torch.from_numpy(perm).cuda()], b["out"])


@pytest.mark.parametrize("base", ["bf16_d128", "fp32_d64"])
def test_tree_extreme_gates(base):
    """Extreme gates on a 40-node tree: alpha at -80 / +-30 / 20, beta at 0 where rho is 1 to the
    last bit and at 1 where alpha is 0, z far into both SiLU tails, against the oracle.  beta = 0
    is kept off the strong decays: along a root path two of them (e^-82 each) would take the state
    below fp32's range, which an fp32 state cannot hold.  In fp32 each node's output is held to 1e-5,
    or to about two ulps of |S| |q| where the readout cancels (_readout_bar)."""
    device, gdn = _mods()
    shape = (W.shape_with(W.TREE_VERIFY, n_pool=2, n_batch=1, n_tok=40) if base == "bf16_d128"
             else W.shape_with(W.TINY_VERIFY, n_pool=2, n_batch=2, n_tok=40))
    say(f"[tree extreme gates] 40 nodes, {base}")
    inp = W.make_tree_inputs(shape, 4)
    rng = np.random.default_rng(9)
    inp["parent"] = np.stack([W.random_tree(rng, shape.n_tok, 8) for _ in range(shape.n_batch)])
    alpha = np.asarray(inp["alpha"]).copy()
    beta = np.asarray(inp["beta"]).copy()
    z = np.asarray(inp["z"]).copy()
    for t in range(shape.n_tok):
        alpha[:, t, :] = (-80.0, 30.0, -30.0, 0.0, 20.0)[t % 5]
        if t % 5 == 0:
            beta[:, t, :] = 0.0
        elif t % 5 == 3:
            beta[:, t, :] = 1.0
    z[:, ::3] = 20.0
    z[:, 1::3] *= -10.0
    # round the edits to the storage dtype, so that the device and the oracle read the same values
    act = shape.act_dtype
    inp.update(alpha=W.round_to(alpha, act), beta=W.round_to(beta, act), z=W.round_to(z, act))
    d = _tree_upload(shape, inp)
    device.verify_tree(d)
    torch.cuda.synchronize()
    _check_tree(shape, inp, d, out_tol=None if base == "bf16_d128" else lambda o: _readout_bar(shape, inp, o))


def _readout_bar(shape, inp, o):
    """Per-(unit, node) output bar of an fp32 tree call: 1e-5 relative to the output, or 1e-7
    (about two fp32 ulps) relative to |S| |q|, whichever is larger.  After a strong decay the state
    is close to rank one (beta v k^T), and o = S q then rests on k.q alone; where q is nearly
    orthogonal to k the readout cancels, and an fp32 dot product is exact only to its ulp relative
    to its operands, not to the cancelled result.  |S| and q come from the oracle's own node states
    and conv windows (parent's conv state rows, then the node's raw row)."""
    cc = ref.tree_conv(shape, inp)
    w = inp["conv_w"].astype(np.float64)
    dk, R = shape.d_k, shape.n_vh // shape.n_kh
    ub, uh = o["units"]
    bar = np.empty((len(ub), shape.n_tok))
    for u in range(len(ub)):
        b, h = int(ub[u]), int(uh[u])
        s = int(inp["slot_ids"][b])
        hk = h // R
        for i in range(shape.n_tok):
            p = int(inp["parent"][b, i])
            prev = inp["conv_state"][s] if p < 0 else cc[b, p]
            win = np.vstack([prev.astype(np.float64), inp["qkv"][b, i].astype(np.float64)[None, :]])
            q = (w.T * win).sum(0)[hk * dk:(hk + 1) * dk]
            S = o["cap"][u, i]
            cond = np.linalg.norm(S) * np.linalg.norm(q) / max(np.linalg.norm(S @ q), 1e-300)
            bar[u, i] = max(tol_for(shape), 1e-7 * cond)
    return bar


def test_tree_captured_in_a_graph_matches_eager():
    """A 130-node tree verify (three launches; the later ones start nodes from captures the earlier
    ones wrote) recorded under stream capture and replayed three times, with new activations and a
    new tree written in place before each replay and the eager call and a synchronisation between
    replays: every replay leaves the eager call's node captures, conv captures and outputs bit for
    bit, and the first matches the oracle."""
    device, gdn = _mods()
    shape = W.shape_with(W.TREE_VERIFY, n_pool=2, n_batch=2, n_tok=130)
    inp = W.make_tree_inputs(shape, 21)
    rng = np.random.default_rng(22)
    inp["parent"] = np.stack([W.random_tree(rng, shape.n_tok, 8) for _ in range(shape.n_batch)])
    eager = _tree_upload(shape, inp, fill_capture=0.0)
    graph = _tree_upload(shape, inp, fill_capture=0.0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        device.verify_tree(graph)
    keys = ("out", "cap_ssm", "cap_conv", "state", "conv_state")
    for r in range(3):
        say(f"[tree graph] replay {r}")
        if r > 0:  # new activations and a new tree, written in place into both sets
            nin = W.make_tree_inputs(shape, 600 + r)
            nin["parent"] = np.stack([W.random_tree(rng, shape.n_tok, 4 + 4 * r) for _ in range(shape.n_batch)])
            for k in ("qkv", "z", "alpha", "beta", "parent"):
                src = torch.from_numpy(np.ascontiguousarray(nin[k])).to(eager[k].dtype).cuda()
                eager[k].copy_(src)
                graph[k].copy_(src)
        graph["out"].fill_(7.0)
        torch.cuda.synchronize()
        device.verify_tree(eager)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in keys:
            assert torch.equal(eager[k], graph[k]), (r, k)
        if r == 0:
            _check_tree(shape, inp, graph)


def test_tree_multiple_roots_and_malformed_parents():
    """Nodes with parent -1 start from the committed state; a malformed parent is treated as -1
    (or rejected with GDN_F_CHECK_INDICES before anything runs)."""
    shape = W.shape_with(W.TINY_VERIFY, n_tok=10, n_pool=2, n_batch=1)
    device, gdn = _mods()
    inp = W.make_tree_inputs(shape, 9)
    par = np.array([[-1, 0, 1, -1, 3, 0, 9, 2, -7, 4]], dtype=np.int32)  # node 6 -> 9, node 8 -> -7
    inp["parent"] = par
    d = _tree_upload(shape, inp)
    device.verify_tree(d)
    torch.cuda.synchronize()
    fixed = dict(inp)
    fixed["parent"] = np.array([[-1, 0, 1, -1, 3, 0, -1, 2, -1, 4]], dtype=np.int32)
    _check_tree(shape, fixed, d)
    e = _tree_upload(shape, inp, flags=gdn.GDN_F_CHECK_INDICES)
    with pytest.raises(gdn.GdnError) as ei:
        device.verify_tree(e)
    assert ei.value.code == gdn.GDN_ERR_RANGE


def test_tree_too_many_nodes_rejected():
    shape = W.shape_with(W.TINY_VERIFY, n_pool=1, n_batch=1, n_tok=1025)
    device, gdn = _mods()
    inp = W.make_tree_inputs(shape, 1)
    d = _tree_upload(shape, inp)
    with pytest.raises(gdn.GdnError) as ei:
        device.verify_tree(d)
    assert ei.value.code == gdn.GDN_ERR_SHAPE


def _kary_parents(n, k):
    return np.array([-1] + [(i - 1) // k for i in range(1, n)], dtype=np.int32)


def test_tree_bushy_shapes_beyond_the_save_slots():
    """Trees whose depth-first walk keeps more branch points open than the kernel has save slots
    (complete binary and ternary trees, a forest of them): a child whose parent's copy was
    evicted re-runs the parent's root path, and every node still matches the oracle."""
    shape = W.shape_with(W.TREE_VERIFY, n_pool=3, n_batch=3, n_tok=63)
    device, _ = _mods()
    inp = W.make_tree_inputs(shape, 4)
    binary = _kary_parents(63, 2)
    ternary = _kary_parents(63, 3)
    forest = np.concatenate([_kary_parents(31, 2), _kary_parents(32, 2) + np.where(
        _kary_parents(32, 2) >= 0, 31, 0)]).astype(np.int32)
    inp["parent"] = np.stack([binary, ternary, forest])
    d = _tree_upload(shape, inp)
    device.verify_tree(d)
    torch.cuda.synchronize()
    _check_tree(shape, inp, d)


def test_tree_bushy_shapes_over_two_launches():
    """A complete binary tree of 127 nodes and a ternary one of 121: their second launch holds
    mostly nodes whose parents are in the first (started from the capture), with branch points
    and re-run paths inside each launch."""
    shape = W.shape_with(W.TREE_VERIFY, n_pool=2, n_batch=2, n_tok=127)
    device, _ = _mods()
    inp = W.make_tree_inputs(shape, 11)
    ternary = np.concatenate([_kary_parents(121, 3), np.arange(120, 126, dtype=np.int32)])
    inp["parent"] = np.stack([_kary_parents(127, 2), ternary])
    d = _tree_upload(shape, inp)
    device.verify_tree(d)
    torch.cuda.synchronize()
    _check_tree(shape, inp, d)
