"""The algorithmic byte and flop models against their hand-derived totals.

Per batch entry the chain verify moves T (C a + 2 H_v a + H_v d_v (a + o)) bytes of inputs and
output, 8 H_v d_v d_k of state (read + write), 24 C of conv state (read + write of 3 rows),
4 T H_v d_v d_k of per-position capture, 4 (3 + T) C of conv window and a 4-byte slot id;
parameters (A_log, dt_bias, conv_w, norm_w) count once.
"""

from gated_deltanet_linear_verify_amd import bytemodel as B
from gated_deltanet_linear_verify_amd import workloads as W


def _verify_by_hand(T, Bn, Hk, Hv, d, a, o):
    C = 2 * Hk * d + Hv * d
    per = (T * (C * a + 2 * Hv * a + Hv * d * (a + o)) + 8 * Hv * d * d + 24 * C
           + 4 * T * Hv * d * d + 4 * (3 + T) * C + 4)
    return Bn * per + 4 * (2 * Hv + 4 * C + d)


def test_verify_bytes_match_hand_totals():
    assert B.verify_bytes(W.TINY_VERIFY) == 466_340 == _verify_by_hand(4, 1, 4, 4, 64, 4, 4)
    assert B.verify_bytes(W.SINGLE_SLOT_VERIFY) == 39_226_116 == _verify_by_hand(16, 1, 16, 32, 128, 2, 2)
    assert B.verify_bytes(W.MULTI_SLOT_VERIFY) == 2_502_165_504 == _verify_by_hand(16, 64, 16, 32, 128, 2, 2)
    # the 2 GiB capture is 85.8% of the multi-slot bytes
    cap = 4 * 64 * 16 * 32 * 128 * 128
    assert cap == 2 * 1024 ** 3
    assert abs(cap / B.verify_bytes(W.MULTI_SLOT_VERIFY) - 0.858) < 1e-3
    # a deferred commit writes neither the 64 slots' states (2 MiB each) nor their conv states
    # (3 rows of 8192 channels): 2,502,165,504 - 64 * (2,097,152 + 98,304)
    assert B.verify_bytes(W.MULTI_SLOT_VERIFY, commit=False) == 2_361_656_320


def test_copy_and_prefill_bytes():
    slot = 4 * (32 * 128 * 128 + 3 * 8192)  # one slot's state + conv state
    assert B.rollback_bytes(W.MULTI_SLOT_VERIFY, 64) == 64 * (2 * slot + 8)  # + slot and index words
    assert B.snapshot_bytes(W.MULTI_SLOT_VERIFY, 64) == 64 * 2 * slot == 281_018_368
    s = W.CHUNKED_PREFILL
    C = s.conv_channels
    hand = (8192 * (C * 2 + 2 * 32 * 2 + 32 * 128 * 4) + 8 * 32 * 128 * 128 + 24 * C
            + 4 * (2 * 32 + 4 * C + 128))
    assert B.prefill_bytes(s) == hand == 274_006_784


def test_tree_bytes_lower_bound():
    s = W.TREE_VERIFY
    C = s.conv_channels
    per = (64 * (C * 2 + 2 * 32 * 2 + 32 * 128 * 4 + 4) + 4 * 32 * 128 * 128 + 12 * C + 4
           + 4 * 64 * 32 * 128 * 128 + 4 * 64 * 3 * C)
    assert B.tree_bytes(s) == 8 * per + 4 * (2 * 32 + 4 * C + 128) == 1_158_613_792


def test_flop_models():
    # ~7 d^2 per (slot, head, token) plus 8 per channel per token for the conv
    assert B.verify_flops(W.MULTI_SLOT_VERIFY) == 64 * 16 * (32 * 7 * 128 * 128 + 8 * 8192)
    # chunked prefill, chunk 64: 4 C d_k + 4 C d_v + 6 d_k d_v + C^2 / 3 per token and head
    assert B.prefill_flops(W.CHUNKED_PREFILL) == 8192 * 32 * (4 * 64 * 128 * 2 + 6 * 128 * 128 + 64 * 64 // 3)
    assert abs(B.prefill_flops(W.CHUNKED_PREFILL) / 1e9 - 43.307) < 1e-3
