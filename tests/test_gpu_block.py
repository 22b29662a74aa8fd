"""GPU: the block's projections (gdn_linear) against the oracle's fp64 x W^T, and a whole GDN
block call (input projections -> verify with capture -> output projection) against the oracle's
block."""

import numpy as np
import pytest

from gated_deltanet_linear_verify_amd import workloads as W
from oracle import block, ref
from tests.gpu_util import half_ulp_bf16, rel_err, say, to_np

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL_F32 = 1e-5  # fp32 accumulation of bf16 products against fp64


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_deltanet_linear_verify_amd import gdn
    gdn.lib()


def _bf16_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda().to(torch.bfloat16).contiguous()


def _operands(M, N, K, seed):
    rng = np.random.default_rng(seed)
    x = W.round_to(rng.standard_normal((M, K)), W.BF16)
    w = W.round_to(rng.normal(0.0, 1.0 / np.sqrt(K), (N, K)), W.BF16)
    return x, w


def _bf16_err(gpu, ref_):
    """max(|gpu - ref| - half a bf16 ulp of ref, 0) / max|ref|: error beyond the output rounding."""
    gpu, ref_ = np.asarray(gpu, np.float64), np.asarray(ref_, np.float64)
    return float(np.max(np.maximum(np.abs(gpu - ref_) - half_ulp_bf16(ref_), 0.0)) / np.max(np.abs(ref_)))


@pytest.mark.parametrize("M,N,K", [(1, 1, 64), (200, 300, 256), (128, 128, 64), (257, 129, 320), (64, 4160, 512)])
def test_linear_fp32_out(M, N, K):
    """Ragged M and N (partial tiles, a single element), several K tiles."""
    from gated_deltanet_linear_verify_amd import gdn
    say(f"[linear] M={M} N={N} K={K}")
    x, w = _operands(M, N, K, seed=M + N + K)
    y = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    gdn.gdn_linear(_bf16_dev(x), _bf16_dev(w), M, N, K, [(0, N, y, N, 0)])
    torch.cuda.synchronize()
    assert rel_err(to_np(y), block.linear(x, w)) < TOL_F32


def test_linear_segments_sigmoid_strides_and_types():
    """Four segments (bf16, bf16 with a row stride wider than the segment, sigmoid fp32, fp32):
    each holds its columns of the product; the padding between rows stays untouched."""
    from gated_deltanet_linear_verify_amd import gdn
    M, K = 70, 192
    widths = [128, 100, 32, 37]
    N = sum(widths)
    x, w = _operands(M, N, K, seed=9)
    want = block.linear(x, w)
    outs = [torch.full((M, 128), 7.0, dtype=torch.bfloat16, device="cuda"),
            torch.full((M, 112), 7.0, dtype=torch.bfloat16, device="cuda"),
            torch.full((M, 32), 7.0, dtype=torch.float32, device="cuda"),
            torch.full((M, 37), 7.0, dtype=torch.float32, device="cuda")]
    segs, n0 = [], 0
    for wd, t, sg in zip(widths, outs, [0, 0, 1, 0]):
        segs.append((n0, n0 + wd, t, t.shape[1], sg))
        n0 += wd
    gdn.gdn_linear(_bf16_dev(x), _bf16_dev(w), M, N, K, segs)
    torch.cuda.synchronize()
    n0 = 0
    for i, (wd, t) in enumerate(zip(widths, outs)):
        got = to_np(t)
        ref_ = want[:, n0:n0 + wd]
        if i == 2:
            ref_ = block.sigmoid(ref_)
        err = _bf16_err(got[:, :wd], ref_) if t.dtype == torch.bfloat16 else rel_err(got[:, :wd], ref_)
        assert err < TOL_F32, (i, err)
        assert np.all(got[:, wd:] == 7.0)
        n0 += wd


def test_linear_full_size_sampled_rows():
    """The 64-slot block's input projection at full size (1024 tokens x 5120 -> 12352 outputs):
    32 sampled rows against the oracle, bf16 outputs as the block stores them."""
    from gated_deltanet_linear_verify_amd import gdn
    s = W.MULTI_SLOT_VERIFY
    M, K = s.n_batch * s.n_tok, W.HIDDEN
    N = s.conv_channels + s.n_vh * s.d_v + 2 * s.n_vh
    x, w = _operands(M, N, K, seed=21)
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    gdn.gdn_linear(_bf16_dev(x), _bf16_dev(w), M, N, K, [(0, N, y, N, 0)])
    torch.cuda.synchronize()
    rows = np.random.default_rng(5).choice(M, 32, replace=False)
    got = to_np(y)[rows]
    assert _bf16_err(got, block.linear(x[rows], w)) < TOL_F32


@pytest.mark.parametrize("name", ["small_d128", "small_d64_ratio1"])
def test_block_against_oracle(name):
    """Input projections, verify with capture (q / k SiLU + unit length), output projection.
    The projections are held to the 1e-5 bar beyond their own bf16 rounding.  The block stores
    its intermediates as bf16 on both sides (projection outputs, the gated output that feeds the
    output projection); where the GPU's fp32 value and the oracle's fp64 value straddle a bf16
    rounding boundary the stored values differ by one ulp (2^-8 relative), so the block's output
    is held to 1e-2 of each entry's largest value, a few such ulps, and the state to 2e-2."""
    from gated_deltanet_linear_verify_amd import device
    base = {"small_d128": W.shape_with(W.MULTI_SLOT_VERIFY, n_kh=2, n_vh=4, n_pool=3, n_batch=2, n_tok=5),
            "small_d64_ratio1": W.shape_with(W.MULTI_SLOT_VERIFY, n_kh=4, n_vh=4, d_k=64, d_v=64, n_pool=2,
                                             n_batch=2, n_tok=3)}[name]
    hidden = 256
    say(f"[block] {name}")
    inp = W.make_block_inputs(base, hidden, seed=31)
    d = device.upload_block(base, inp)
    device.block_step(d)
    torch.cuda.synchronize()
    r = block.block_verify(base, inp)
    p = r["proj"]
    B, T, Hv, dv = base.n_batch, base.n_tok, base.n_vh, base.d_v
    # the projections: beyond their own bf16 rounding, as the product
    assert _bf16_err(to_np(d["qkv"]), block.linear(inp["x"], inp["w_qkv"])) < TOL_F32
    assert _bf16_err(to_np(d["beta"]), block.sigmoid(block.linear(inp["x"], inp["w_beta"]))) < TOL_F32
    flips = np.mean(to_np(d["qkv"]) != p["qkv"])
    say(f"  qkv elements one bf16 rounding apart: {flips:.4f}")
    y = to_np(d["y"]).astype(np.float64)
    for b in range(B):
        err = rel_err(y[b], r["y"][b])
        say(f"  entry {b}: block output rel err {err:.2e}")
        assert err < 1e-2
    st = to_np(d["state"])
    for b in range(B):
        s_ = int(inp["slot_ids"][b])
        for h in range(Hv):
            assert rel_err(st[s_, h], r["state"][s_, h]) < 2e-2
