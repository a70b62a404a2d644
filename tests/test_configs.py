"""Algorithmic accounting of the five workloads against closed-form counts."""
import pytest

from ring_causal_attention_amd import configs, synth

pytestmark = pytest.mark.cpu


def test_pair_and_flop_counts():
    W = configs.WORKLOADS
    # full causal: L(L+1)/2 pairs per head
    assert W["llama7b_fwd_L32768"].visible_pairs() == 32 * 32768 * 32769 // 2 == 17_180_393_472
    assert W["llama7b_fwd_L32768"].fwd_flop() == 8_796_361_457_664
    assert W["causal_fp32_L1024"].visible_pairs() == 4 * 524_800
    # ring share at shard 40 of 64: 40 full shards + the diagonal shard
    assert W["ring_share_1M"].visible_pairs() == 8 * (40 * 16384 ** 2 + 16384 * 16385 // 2) == 86_973_153_280
    # training step: forward 4D + backward 10D per pair
    t = W["train_step_L32768"]
    assert t.total_flop() == 14 * 128 * 17_180_393_472
    assert W["ring_share_1M"].ring_order()[:3] == [40, 39, 38] and W["ring_share_1M"].ring_order()[40:42] == [0, 63]


def test_packed_segments_seed_1003():
    w = configs.WORKLOADS["packed_L65536"]
    lens = w.segment_lengths()
    assert sum(lens) == 65536 and all(256 <= n <= 8192 for n in lens[:-1])
    assert lens[:4] == [2888, 5775, 2136, 4474] and lens[-1] == 240 and len(lens) == 17
    assert w.visible_pairs() == 5_673_673_632


def test_bf16_rounding_is_rne():
    import numpy as np
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 1.0 + 2 ** -8 + 2 ** -20], dtype=np.float32)
    r = synth.round_to_bf16(x)
    # bf16 keeps 7 fraction bits; ties go to even: 1+2^-8 -> 1, 1+3*2^-8 -> 1+2^-6
    assert r[0] == 1.0 and r[1] == 1.0 and r[2] == np.float32(1.0 + 2 ** -6) and r[3] == -2.5
    assert r[4] == np.float32(1.0 + 2 ** -7)  # above the tie: rounds up
