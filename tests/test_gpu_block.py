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


@pytest.mark.parametrize("M,N,K", [(1, 1, 64), (200, 300, 256), (128, 128, 64), (257, 129, 320), (64, 4160, 512),
                                   (1100, 10000, 320),
                                   # few rows: one-wave 16 x 16 or 32 x 16 tiles, four buffered k
                                   # tiles (one k tile at K = 64, three at 192)
                                   (7, 1000, 192), (16, 17, 128), (16, 5120, 4096), (16, 12352, 512),
                                   (24, 700, 320), (48, 5120, 4096),
                                   # 65 - 1023 rows: 64 x 128 tiles (uneven x transfers), 64 x 64
                                   # tiles with three buffered k tiles (at K = 128 and 192 fewer k
                                   # tiles than buffers), 32 x 64 tiles
                                   (300, 9000, 256), (130, 9000, 192), (200, 5000, 128), (100, 3000, 320)])
def test_linear_fp32_out(M, N, K):
    """Ragged M and N (partial tiles, a single element), several K tiles; the last shape has enough
    256 x 256 tiles (5 x 40) to take that tiling, with partial tiles along both M and N."""
    from gated_deltanet_linear_verify_amd import gdn
    say(f"[linear] M={M} N={N} K={K}")
    x, w = _operands(M, N, K, seed=M + N + K)
    y = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    gdn.gdn_linear(_bf16_dev(x), _bf16_dev(w), M, N, K, [(0, N, y, N, 0)])
    torch.cuda.synchronize()
    assert rel_err(to_np(y), block.linear(x, w)) < TOL_F32


@pytest.mark.parametrize("M", [70, 12])
def test_linear_segments_sigmoid_strides_and_types(M):
    """Four segments (bf16, bf16 with a row stride wider than the segment, sigmoid fp32, fp32):
    each holds its columns of the product; the padding between rows stays untouched (at 70 rows on
    32 x 64 tiles, at 12 on 16 x 16)."""
    from gated_deltanet_linear_verify_amd import gdn
    K = 192
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
    """Input projections, verify with capture (q / k SiLU + unit length), output projection, each
    stage held to its own bar on the values the previous stage actually stored:
    * the four input projections against the oracle's fp64 x W^T, 1e-5 beyond their bf16 rounding;
    * the verify against the oracle run on the GPU's stored bf16 qkv / z / beta / alpha: state and
      every capture position 2e-3, the gated output 2e-3 beyond its own bf16 rounding, the conv
      window and conv state bit for bit;
    * the output projection against the oracle's fp64 product of the GPU's stored bf16 gated
      output, 1e-5 beyond its bf16 rounding.
    Chaining the stages on the oracle side alone would compare bf16 intermediates that can sit one
    rounding apart (a value whose fp32 and fp64 forms straddle a bf16 rounding boundary); the
    stage-wise form holds every arithmetic step to the stated tolerance instead."""
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
    B, T, Hv, dv = base.n_batch, base.n_tok, base.n_vh, base.d_v
    # stage 1: the projections, beyond their own bf16 rounding
    x = inp["x"]
    assert _bf16_err(to_np(d["qkv"]), block.linear(x, inp["w_qkv"]).reshape(B, T, -1)) < TOL_F32
    assert _bf16_err(to_np(d["z"]), block.linear(x, inp["w_z"]).reshape(B, T, Hv, dv)) < TOL_F32
    assert _bf16_err(to_np(d["beta"]), block.sigmoid(block.linear(x, inp["w_beta"])).reshape(B, T, Hv)) < TOL_F32
    assert _bf16_err(to_np(d["alpha"]), block.linear(x, inp["w_alpha"]).reshape(B, T, Hv)) < TOL_F32
    # stage 2: the verify, on the inputs the projections stored
    layer = dict(inp)
    for k in ("qkv", "z", "alpha", "beta"):
        layer[k] = to_np(d[k])
    o = ref.verify_pool(base, layer, flags=ref.F_QK_NORM_SILU)
    st, cap, out = to_np(d["state"]), to_np(d["cap_ssm"]), to_np(d["out"])
    worst = {"state": 0.0, "cap": 0.0, "out": 0.0}
    for b in range(B):
        s_ = int(inp["slot_ids"][b])
        for h in range(Hv):
            worst["state"] = max(worst["state"], rel_err(st[s_, h], o["state"][s_, h]))
            worst["out"] = max(worst["out"], _bf16_err(out[b, :, h], o["out"][b, :, h]))
            for t in range(T):
                worst["cap"] = max(worst["cap"], rel_err(cap[s_, t, h], o["cap_ssm"][s_, t, h]))
        np.testing.assert_array_equal(to_np(d["cap_conv"])[s_], o["cap_conv"][s_])
    np.testing.assert_array_equal(to_np(d["conv_state"]), o["conv_state"])
    say(f"  verify stage on the stored projections: {worst}")
    for k, v in worst.items():
        assert v <= 2e-3, (k, v)
    # stage 3: the output projection of the stored gated output
    y = to_np(d["y"])
    want = block.linear(out.reshape(B * T, Hv * dv), inp["w_out"]).reshape(B, T, -1)
    err = _bf16_err(y, want)
    say(f"  output projection beyond bf16 rounding: {err:.2e}")
    assert err < TOL_F32
    # for information: the whole block against the oracle's own chain of bf16 intermediates
    r = block.block_verify(base, inp)
    say(f"  end to end (bf16 intermediates on each side): {rel_err(y, r['y']):.2e}")


def test_linear_out_projection_full_size_sampled_rows():
    """The 64-slot block's output projection at full size (1024 tokens x 4096 -> 5120, the
    128 x 128 tiling): 32 sampled rows against the oracle, bf16 outputs."""
    from gated_deltanet_linear_verify_amd import gdn
    s = W.MULTI_SLOT_VERIFY
    M, K, N = s.n_batch * s.n_tok, s.n_vh * s.d_v, W.HIDDEN
    x, w = _operands(M, N, K, seed=22)
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    gdn.gdn_linear(_bf16_dev(x), _bf16_dev(w), M, N, K, [(0, N, y, N, 0)])
    torch.cuda.synchronize()
    rows = np.random.default_rng(6).choice(M, 32, replace=False)
    assert _bf16_err(to_np(y)[rows], block.linear(x[rows], w)) < TOL_F32
