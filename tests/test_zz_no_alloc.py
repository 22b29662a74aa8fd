"""GPU: gdn_prefill_noalloc (the prefill whose workspace is the library's static device array)
against gdn_prefill with a caller workspace, through the C ABI, on two calls in a row, the second
with a smaller input."""

import numpy as np
import pytest

from gated_deltanet_linear_verify_amd import workloads as W
from tests.gpu_util import out_err, rel_err, say, to_np, tol_for

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_deltanet_linear_verify_amd import gdn
    gdn.lib()


def _noalloc(d, stream=None):
    from gated_deltanet_linear_verify_amd import gdn
    T = d["qkv"].shape[1]
    gdn.gdn_prefill_noalloc(d["dims"], d["state"], d["conv_state"], d["qkv"], d["z"], d["alpha"], d["beta"],
                            d["A_log"], d["dt_bias"], d["conv_w"], d["norm_w"], d["out"], T, d["slot"], stream)


def test_noalloc_prefill_equals_workspace_prefill_twice():
    """Two calls in a row on the 8192-token workload's dims: 2500 tokens (three pieces of the static
    scratch: 960 + 960 + 580), then 130 tokens (one piece, into a scratch that still holds the first
    call's contents).  Each against gdn_prefill on the same inputs: out, state and conv state within
    the stated tolerance, and here bit for bit (the pieces are whole 64-token chunks, so every chunk
    and every state carried between pieces is the same fp32 arithmetic)."""
    from gated_deltanet_linear_verify_amd import device
    for n_tok, seed in ((2500, 11), (130, 12)):
        shape = W.shape_with(W.CHUNKED_PREFILL, n_tok=n_tok, n_pool=2)
        inp = W.make_inputs(shape, seed, weak_decay=True)
        say(f"[prefill no-alloc] {n_tok} tokens, slot {int(inp['slot_ids'][0])}")
        ref_d = device.upload(shape, inp, capture=False)
        device.prefill(ref_d)
        d = device.upload(shape, inp, capture=False)
        _noalloc(d)
        torch.cuda.synchronize()
        s = d["slot"]
        tol = tol_for(shape)
        es = rel_err(to_np(d["state"][s]), to_np(ref_d["state"][s]))
        eo = max(out_err(shape, to_np(d["out"])[0, :, h], to_np(ref_d["out"])[0, :, h]) for h in range(shape.n_vh))
        say(f"  state rel err {es:.2e}, out {eo:.2e}; bitwise: state {torch.equal(d['state'], ref_d['state'])}, "
            f"out {torch.equal(d['out'], ref_d['out'])}")
        assert es <= tol and eo <= tol
        assert torch.equal(d["state"], ref_d["state"])
        assert torch.equal(d["out"], ref_d["out"])
        assert torch.equal(d["conv_state"], ref_d["conv_state"])
        # the other slot of the pool is untouched
        o = 1 - s
        np.testing.assert_array_equal(to_np(d["state"][o]), inp["state"][o])


def test_noalloc_prefill_rejects_bad_arguments_without_launching():
    from gated_deltanet_linear_verify_amd import device, gdn
    shape = W.shape_with(W.CHUNKED_PREFILL, n_tok=64)
    d = device.upload(shape, W.make_inputs(shape, 1), capture=False)
    with pytest.raises(gdn.GdnError) as ei:
        _noalloc(dict(d, slot=5))
    assert ei.value.code == gdn.GDN_ERR_RANGE
