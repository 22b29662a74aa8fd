"""The seeded input generators: determinism, shapes, and the stated distributions."""

import numpy as np
import pytest

from gated_deltanet_linear_verify_amd import workloads as W


@pytest.mark.parametrize("name", ["tiny_verify", "single_slot_verify"])
def test_generator_is_deterministic(name):
    shape = W.WORKLOADS[name]
    a = W.make_inputs(shape, 0)
    b = W.make_inputs(shape, 0)
    c = W.make_inputs(shape, 1)
    assert W.digest(a) == W.digest(b)
    assert W.digest(a) != W.digest(c)


def test_shapes_and_recipe_single_slot():
    s = W.SINGLE_SLOT_VERIFY
    inp = W.make_inputs(s, 0)
    C = s.conv_channels
    assert C == 8192
    assert inp["qkv"].shape == (1, 16, C)
    assert inp["z"].shape == (1, 16, 32, 128)
    assert inp["alpha"].shape == inp["beta"].shape == (1, 16, 32)
    assert inp["state"].shape == (1, 32, 128, 128)
    assert inp["conv_state"].shape == (1, 3, C)
    assert inp["conv_w"].shape == (C, 4)
    # q and k head slices have unit length (up to bf16 rounding), v does not
    nqk = s.n_kh * s.d_k
    qk = inp["qkv"][0, :, :2 * nqk].reshape(16, 2 * s.n_kh, s.d_k).astype(np.float64)
    np.testing.assert_allclose(np.linalg.norm(qk, axis=-1), 1.0, atol=2e-2)
    # bf16 activations: values survive a bf16 round trip unchanged
    import torch
    for k in ("qkv", "z", "alpha", "beta"):
        t = torch.from_numpy(inp[k])
        assert torch.equal(t.to(torch.bfloat16).to(torch.float32), t)
    assert np.all((inp["beta"] > 0) & (inp["beta"] < 1))
    assert np.all((inp["A_log"] >= 0) & (inp["A_log"] <= 1))


def test_multi_slot_permutation_and_trims():
    s = W.shape_with(W.MULTI_SLOT_VERIFY, d_k=8, d_v=8)
    inp = W.make_inputs(s, 0)
    assert sorted(inp["slot_ids"].tolist()) == list(range(64))
    assert np.all((inp["trims"] >= 0) & (inp["trims"] < 16))


def test_random_tree_shape():
    rng = np.random.default_rng(0)
    for _ in range(20):
        p = W.random_tree(rng, 64)
        assert p[0] == -1
        assert np.all(p[1:] >= 0) and np.all(p[1:] < np.arange(1, 64))
        assert W.tree_depths(p).max() <= W.TREE_MAX_DEPTH
        a = W.tree_accept(rng, p)
        assert 0 <= a < 64


def test_chain_parents():
    np.testing.assert_array_equal(W.chain_parents(4), [-1, 0, 1, 2])
