"""lwm_ring_step: a ring of KV shards folded into (O, lse) equals full attention (oracle)."""
import numpy as np
import pytest
import torch

import oracle
from ring_causal_attention_amd import lwm, path, synth
from tests.gpu_utils import BF16_MAX_ABS, BF16_MEAN_ABS, LSE_BF16, dev, errors, exact_host, host, need_gpu, note, seg_dev

pytestmark = pytest.mark.gpu


def shards_case(seed, n_shards, shard, Lq, r, H=2, order=None):
    B = 1
    q = synth.normal(seed, "q", (B, Lq, H, 128))
    k = [synth.normal(seed, "k", (B, shard, H, 128), shard=j) for j in range(n_shards)]
    v = [synth.normal(seed, "v", (B, shard, H, 128), shard=j) for j in range(n_shards)]
    q_off = r * shard
    order = order if order is not None else [(r - s) % n_shards for s in range(n_shards)]
    return q, k, v, q_off, order


@pytest.mark.parametrize("n_shards,shard,r", [(6, 64, 3), (5, 100, 4), (4, 129, 0), (8, 200, 5)])
def test_ring_equals_full_attention(n_shards, shard, r):
    need_gpu()
    note(f"ring n_shards={n_shards} shard={shard} r={r}")
    q, k, v, q_off, order = shards_case(1000 + shard, n_shards, shard, shard, r)
    kd = [dev(x, "bf16") for x in k]
    vd = [dev(x, "bf16") for x in v]
    o, o_acc, lse = path.ring_forward(dev(q, "bf16"), kd, vd, order, shard, q_off)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.attention_fwd(exact_host(q, "bf16"), np.concatenate([exact_host(x, "bf16") for x in k], 1),
                                        np.concatenate([exact_host(x, "bf16") for x in v], 1), None, None, q_off, 0, True)
    mx, mean = errors(host(o), ref_o)
    assert mx <= BF16_MAX_ABS and mean <= BF16_MEAN_ABS, (mx, mean)
    mx32, _ = errors(host(o_acc), ref_o)
    assert mx32 <= 1e-2, mx32
    assert np.max(np.abs(host(lse) - ref_l)) <= LSE_BF16


def test_ring_order_invariance():
    need_gpu()
    note("ring order invariance")
    q, k, v, q_off, order = shards_case(1100, 6, 96, 96, 4)
    qd = dev(q, "bf16")
    kd = [dev(x, "bf16") for x in k]
    vd = [dev(x, "bf16") for x in v]
    a, _, la = path.ring_forward(qd, kd, vd, order, 96, q_off)
    b, _, lb = path.ring_forward(qd, kd, vd, order[::-1], 96, q_off)
    torch.cuda.synchronize()
    assert np.max(np.abs(host(a) - host(b))) <= 2e-2 and np.max(np.abs(host(la) - host(lb))) <= LSE_BF16


def test_unvisited_rows_keep_state_bitwise():
    need_gpu()
    note("ring state untouched by a shard that no row sees / rows that see nothing")
    B, Lq, H, S = 1, 100, 2, 64
    q = dev(synth.normal(1200, "q", (B, Lq, H, 128)), "bf16")
    k = dev(synth.normal(1200, "k", (B, S, H, 128)), "bf16")
    v = dev(synth.normal(1200, "v", (B, S, H, 128)), "bf16")
    o_acc = torch.randn((B, Lq, H, 128), device="cuda")
    lse = torch.randn((B, H, Lq), device="cuda")
    o0, l0 = o_acc.clone(), lse.clone()
    # the shard starts after every query: nothing visible
    lwm.lwm_ring_step(q, k, v, o_acc, lse, q_offset=1000, k_offset=5000)
    torch.cuda.synchronize()
    assert torch.equal(o_acc, o0) and torch.equal(lse, l0)
    # the shard starts at query 60: rows 0..59 see nothing and keep their state
    lwm.lwm_ring_step(q, k, v, o_acc, lse, q_offset=1000, k_offset=1060)
    torch.cuda.synchronize()
    assert torch.equal(o_acc[:, :60], o0[:, :60]) and torch.equal(lse[:, :, :60], l0[:, :, :60])
    assert not torch.equal(o_acc[:, 60:], o0[:, 60:])


def test_ring_with_packing_segments():
    need_gpu()
    note("ring step with segment ids")
    n, S, H = 4, 80, 2
    Ltot = n * S
    seg = synth.random_segment_ids(1300, 1, Ltot, 70)
    q_all = synth.normal(1300, "q", (1, Ltot, H, 128))
    k_all = synth.normal(1300, "k", (1, Ltot, H, 128))
    v_all = synth.normal(1300, "v", (1, Ltot, H, 128))
    r = 3
    qs = slice(r * S, (r + 1) * S)
    qd = dev(q_all[:, qs], "bf16")
    kd = [dev(k_all[:, j * S:(j + 1) * S], "bf16") for j in range(n)]
    vd = [dev(v_all[:, j * S:(j + 1) * S], "bf16") for j in range(n)]
    sk = [seg_dev(seg[:, j * S:(j + 1) * S]) for j in range(n)]
    o, _, lse = path.ring_forward(qd, kd, vd, [3, 2, 1, 0], S, r * S, seg_q=seg_dev(seg[:, qs]), seg_k_shards=sk)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.attention_fwd(exact_host(q_all[:, qs], "bf16"), exact_host(k_all, "bf16"),
                                        exact_host(v_all, "bf16"), seg[:, qs], seg, r * S, 0, True)
    mx, mean = errors(host(o), ref_o)
    assert mx <= BF16_MAX_ABS and mean <= BF16_MEAN_ABS
