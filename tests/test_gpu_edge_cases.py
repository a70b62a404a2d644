"""Degenerate inputs of the backward, the backward ring step and the fused-RoPE calls: empty query
or key sides, zero batch or heads, query rows that see no key, shards wholly in the causal future.
Outputs are poisoned with NaN first, so every element a call must write is checked written."""
import numpy as np
import pytest
import torch

import oracle
from ring_causal_attention_amd import lwm, synth
from tests.gpu_utils import GRAD_REL_FRO, dev, exact_host, host, need_gpu, note, rel_fro

pytestmark = pytest.mark.gpu


def nan_like(t, dtype=None):
    return torch.full(t.shape, float("nan"), dtype=dtype or t.dtype, device=t.device)


@pytest.mark.parametrize("Lq,Lk", [(0, 10), (10, 0), (0, 0)])
def test_backward_with_an_empty_side(Lq, Lk):
    need_gpu()
    note(f"bwd empty side Lq={Lq} Lk={Lk}")
    q = dev(synth.normal(3000, "q", (1, Lq, 2, 128)), "bf16")
    k = dev(synth.normal(3000, "k", (1, Lk, 2, 128)), "bf16")
    v = dev(synth.normal(3000, "v", (1, Lk, 2, 128)), "bf16")
    do = dev(synth.normal(3000, "do", (1, Lq, 2, 128)), "bf16")
    o, lse = lwm.lwm_blockattn_fwd(q, k, v)
    dq, dk, dv = nan_like(q), nan_like(k), nan_like(v)
    lwm.lwm_blockattn_bwd(q, k, v, o, lse, do, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    # no pair is visible: every gradient that exists is exactly zero
    for g in (dq, dk, dv):
        assert g.numel() == 0 or float(g.float().abs().max()) == 0.0


@pytest.mark.parametrize("shape", [(0, 64, 2, 128), (1, 64, 0, 128)])
def test_zero_batch_or_heads_is_a_no_op(shape):
    need_gpu()
    note(f"zero batch / heads {shape}")
    x = torch.zeros(shape, dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((shape[0], shape[2], shape[1]), dtype=torch.float32, device="cuda")
    o, _ = lwm.lwm_blockattn_fwd(x, x, x)
    lwm.lwm_blockattn_bwd(x, x, x, o, lse, x)
    lwm.lwm_blockattn_fwd_rope(x, x, x, 1e6)
    lwm.lwm_blockattn_bwd_rope(x, x, x, o, lse, x, 1e6)
    acc = torch.zeros(shape, dtype=torch.float32, device="cuda")
    lwm.lwm_ring_step_bwd(x, x, x, o, lse, x, acc, acc.clone(), acc.clone())
    torch.cuda.synchronize()


def test_backward_rows_that_see_no_key():
    need_gpu()
    note("bwd: query rows 0..49 see no key (k_offset = 50)")
    L, H = 200, 2
    q, k, v, do = (synth.normal(3100, t, (1, L, H, 128)) for t in ("q", "k", "v", "do"))
    qd, kd, vd, dod = (dev(x, "bf16") for x in (q, k, v, do))
    o, lse = lwm.lwm_blockattn_fwd(qd, kd, vd, q_offset=0, k_offset=50)
    dq, dk, dv = nan_like(qd), nan_like(kd), nan_like(vd)
    lwm.lwm_blockattn_bwd(qd, kd, vd, o, lse, dod, q_offset=0, k_offset=50, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    gq = host(dq)
    assert np.all(gq[:, :50] == 0.0)
    rdq, rdk, rdv = oracle.attention_bwd(*(exact_host(x, "bf16") for x in (q, k, v, do)), None, None, 0, 50, True)
    for g, r in ((gq, rdq), (host(dk), rdk), (host(dv), rdv)):
        assert np.all(np.isfinite(g)) and rel_fro(g, r) <= GRAD_REL_FRO


def test_ring_step_bwd_adds_nothing_for_empty_or_future_shards():
    need_gpu()
    note("backward ring step: empty shard and a shard wholly in the causal future")
    Lq, S, H = 128, 96, 2
    q, do = (dev(synth.normal(3200, t, (1, Lq, H, 128)), "bf16") for t in ("q", "do"))
    k, v = (dev(synth.normal(3200, t, (1, S, H, 128)), "bf16") for t in ("k", "v"))
    o, lse = lwm.lwm_blockattn_fwd(q, k, v, q_offset=S, k_offset=0)
    f32 = dict(dtype=torch.float32, device="cuda")
    dq_acc = torch.randn((1, Lq, H, 128), **f32)
    dk_acc, dv_acc = torch.randn((1, S, H, 128), **f32), torch.randn((1, S, H, 128), **f32)
    before = [t.clone() for t in (dq_acc, dk_acc, dv_acc)]
    # keys starting after the block's last query: nothing is visible
    lwm.lwm_ring_step_bwd(q, k, v, o, lse, do, dq_acc, dk_acc, dv_acc, q_offset=S, k_offset=S + Lq)
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip((dq_acc, dk_acc, dv_acc), before))
    # an empty shard
    e = torch.zeros((1, 0, H, 128), dtype=torch.bfloat16, device="cuda")
    ea = torch.zeros((1, 0, H, 128), **f32)
    lwm.lwm_ring_step_bwd(q, e, e, o, lse, do, dq_acc, ea, ea.clone(), q_offset=S, k_offset=0)
    torch.cuda.synchronize()
    assert torch.equal(dq_acc, before[0])


@pytest.mark.parametrize("Lq,Lk", [(0, 10), (10, 0)])
def test_fused_rope_with_an_empty_side(Lq, Lk):
    need_gpu()
    note(f"fused rope empty side Lq={Lq} Lk={Lk}")
    q = dev(synth.normal(3300, "q", (1, Lq, 2, 128)), "bf16")
    k = dev(synth.normal(3300, "k", (1, Lk, 2, 128)), "bf16")
    v = dev(synth.normal(3300, "v", (1, Lk, 2, 128)), "bf16")
    do = dev(synth.normal(3300, "do", (1, Lq, 2, 128)), "bf16")
    o, lse, qr, kr = lwm.lwm_blockattn_fwd_rope(q, k, v, 1e6)
    dq, dk, dv = lwm.lwm_blockattn_bwd_rope(qr, kr, v, o, lse, do, 1e6, dq=nan_like(q), dk=nan_like(k),
                                            dv=nan_like(v))
    torch.cuda.synchronize()
    if Lq:
        assert float(o.float().abs().sum()) == 0.0 and bool(torch.isneginf(lse).all())
        assert torch.equal(qr, lwm.lwm_rope_apply(q, theta=1e6))
    if Lk:
        assert torch.equal(kr, lwm.lwm_rope_apply(k, theta=1e6))
    for g in (dq, dk, dv):
        assert g.numel() == 0 or float(g.float().abs().max()) == 0.0


def test_fused_rope_rows_that_see_no_key():
    need_gpu()
    note("fused rope: query rows 0..63 see no key (k_offset = 64)")
    L, H, theta = 190, 2, 1e6
    q, k, v, do = (synth.normal(3400, t, (1, L, H, 128)) for t in ("q", "k", "v", "do"))
    qd, kd, vd, dod = (dev(x, "bf16") for x in (q, k, v, do))
    o, lse, qr, kr = lwm.lwm_blockattn_fwd_rope(qd, kd, vd, theta, q_offset=0, k_offset=64, k_pos_offset=64)
    dq, dk, dv = lwm.lwm_blockattn_bwd_rope(qr, kr, vd, o, lse, dod, theta, q_offset=0, k_offset=64,
                                            k_pos_offset=64, dq=nan_like(qd), dk=nan_like(kd), dv=nan_like(vd))
    torch.cuda.synchronize()
    assert np.all(host(o)[:, :64] == 0.0) and bool(torch.isneginf(lse[:, :, :64]).all())
    assert np.all(host(dq)[:, :64] == 0.0)
    pos_q, pos_k = oracle.positions(1, L, 0), oracle.positions(1, L, 64)
    ro, rl, rdq, rdk, rdv = oracle.training_step(*(exact_host(x, "bf16") for x in (q, k, v, do)), pos_q, pos_k,
                                                 theta, "half", None, None, 0, 64, True)
    assert np.max(np.abs(host(o) - ro)) <= 2e-2
    for g, r in ((dq, rdq), (dk, rdk), (dv, rdv)):
        gg = host(g)
        assert np.all(np.isfinite(gg)) and rel_fro(gg, r) <= GRAD_REL_FRO
