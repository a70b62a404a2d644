"""lwm_ring_step_bwd: KV shards visited backward around the ring, each adding its share of the
gradients, give the gradients of attention over all keys ("开源巨兽LWM：如何用RingAttention撬动百万Token
多模态世界", section 3.1: the query block stays while key/value blocks travel the ring).

Three checks per case:
* end to end: dQ, and dK / dV with the shards concatenated, against the oracle's gradients of
  attention over all keys, from the exact inputs and the oracle's own O (the definition);
* the same ring against the library's single-call backward over the concatenated keys, given the
  same forward results (equal up to float32 summation order and the final bf16 rounding);
* per shard: each step against the oracle's backward ring step on the O and lse the GPU forward
  produced (a unit check of one step: the step is a function of that O and lse).
"""
import numpy as np
import pytest
import torch

import oracle
from ring_causal_attention_amd import lwm, path, synth
from tests.gpu_utils import (BF16_MAX_ABS, BF16_MEAN_ABS, GRAD_REL_FRO, dev, errors, exact_host, host, need_gpu, note,
                             rel_fro, report, seg_dev)

pytestmark = pytest.mark.gpu


def ring_bwd_case(seed, n_shards, shard, Lq, q_off, H=2, segs=False, order=None):
    """GPU forward + backward ring: end to end against the oracle over all keys, against the
    single-call backward, and step by step against the oracle's backward ring step."""
    Ltot = n_shards * shard
    q = synth.normal(seed, "q", (1, Lq, H, 128))
    do = synth.normal(seed, "do", (1, Lq, H, 128))
    k_all = synth.normal(seed, "k", (1, Ltot, H, 128))
    v_all = synth.normal(seed, "v", (1, Ltot, H, 128))
    seg = synth.random_segment_ids(seed, 1, max(Ltot, q_off + Lq), 70) if segs else None
    seg_q = None if seg is None else seg[:, q_off:q_off + Lq]
    seg_k = [None if seg is None else seg[:, j * shard:(j + 1) * shard] for j in range(n_shards)]
    home = min(n_shards - 1, q_off // shard)
    order = order if order is not None else [(home - s) % n_shards for s in range(n_shards)]

    qd, dod = dev(q, "bf16"), dev(do, "bf16")
    kd = [dev(k_all[:, j * shard:(j + 1) * shard], "bf16") for j in range(n_shards)]
    vd = [dev(v_all[:, j * shard:(j + 1) * shard], "bf16") for j in range(n_shards)]
    sqd = None if seg is None else seg_dev(seg_q)
    skd = None if seg is None else [seg_dev(x) for x in seg_k]
    o, _, lse = path.ring_forward(qd, kd, vd, order, shard, q_off, seg_q=sqd, seg_k_shards=skd)
    dq_acc, dk_acc, dv_acc = path.ring_backward(qd, kd, vd, o, lse, dod, order, shard, q_off, seg_q=sqd,
                                                seg_k_shards=skd)
    torch.cuda.synchronize()

    qe, doe, ke, ve = (exact_host(x, "bf16") for x in (q, do, k_all, v_all))
    seg_k_all = None if seg is None else seg[:, :Ltot]
    # the ring forward against attention over all keys
    ex_o, _ = oracle.attention_fwd(qe, ke, ve, seg_q, seg_k_all, q_off, 0, True)
    mx, mean = errors(host(o), ex_o)
    assert mx <= BF16_MAX_ABS and mean <= BF16_MEAN_ABS, ("o", mx, mean)

    def concat(acc):  # shards in key order; a shard the ring skipped contributes zeros
        return np.concatenate([host(acc[j]) if j in acc else np.zeros((1, shard, H, 128)) for j in range(n_shards)],
                              axis=1)

    got_dq, got_dk, got_dv = host(dq_acc), concat(dk_acc), concat(dv_acc)
    # (1) end to end: the gradients of attention over all keys (exact inputs, the oracle's own O)
    ex_dq, ex_dk, ex_dv = oracle.attention_bwd(qe, ke, ve, doe, seg_q, seg_k_all, q_off, 0, True)
    for name, got, ref in (("dq", got_dq, ex_dq), ("dk", got_dk, ex_dk), ("dv", got_dv, ex_dv)):
        e = rel_fro(got, ref)
        assert e <= GRAD_REL_FRO, ("end to end", name, e)
    # (2) the library's single-call backward over the concatenated keys, same forward results
    k_cat, v_cat = torch.cat(kd, dim=1), torch.cat(vd, dim=1)
    sk_cat = None if seg is None else seg_dev(seg_k_all)
    mdq, mdk, mdv = lwm.lwm_blockattn_bwd(qd, k_cat, v_cat, o, lse, dod, seg_q=sqd, seg_k=sk_cat, q_offset=q_off,
                                          k_offset=0)
    torch.cuda.synchronize()
    for name, got, ref in (("dq", got_dq, host(mdq)), ("dk", got_dk, host(mdk)), ("dv", got_dv, host(mdv))):
        e = rel_fro(got, ref)
        assert e <= 5e-3, ("vs single-call backward", name, e)
    # (3) per shard, on the O (bf16) and lse the GPU forward produced: in a shard that a query
    # reaches through only a few keys, dP - delta cancels, so the forward's rounding of O weighs
    # more in that shard's share than in the whole gradient
    ref_o, ref_l = host(o), host(lse)
    ref_dq = np.zeros_like(qe)
    for j in range(n_shards):
        sl = slice(j * shard, (j + 1) * shard)
        dqj, dkj, dvj = oracle.ring_step_bwd(qe, ke[:, sl], ve[:, sl], ref_o, ref_l, doe, seg_q, seg_k[j], q_off,
                                             j * shard, True)
        ref_dq += dqj
        if j in dk_acc:
            for name, got, ref in (("dk", dk_acc[j], dkj), ("dv", dv_acc[j], dvj)):
                if np.any(ref):
                    e = rel_fro(host(got), ref)
                    assert e <= GRAD_REL_FRO, (name, j, e)
                else:
                    assert not bool(got.any()), (name, j)
        else:
            assert not np.any(dkj) and not np.any(dvj), j  # skipped shards add nothing
    e = rel_fro(got_dq, ref_dq)
    assert e <= GRAD_REL_FRO, ("dq", e)
    report(f"ring_bwd n{n_shards}x{shard} q{Lq}@{q_off}{'s' if segs else ''}", dq_rel_fro=rel_fro(got_dq, ex_dq),
           dk_rel_fro=rel_fro(got_dk, ex_dk), dv_rel_fro=rel_fro(got_dv, ex_dv))
    return dq_acc, dk_acc, dv_acc


@pytest.mark.parametrize("n_shards,shard,Lq,q_off", [(6, 128, 160, 3 * 128 + 37), (5, 100, 100, 400),
                                                     (4, 129, 129, 0), (3, 64, 200, 150)])
def test_ring_backward_equals_full_gradients(n_shards, shard, Lq, q_off):
    need_gpu()
    note(f"ring backward n_shards={n_shards} shard={shard} Lq={Lq} q_off={q_off}")
    ring_bwd_case(2000 + shard, n_shards, shard, Lq, q_off)


def test_ring_backward_with_packing_segments():
    need_gpu()
    note("ring backward with segment ids")
    ring_bwd_case(2100, 4, 96, 96, 3 * 96, segs=True)


def test_ring_backward_order_and_accumulation():
    need_gpu()
    note("ring backward: visiting order does not matter; a second pass adds the same again")
    n, S, Lq, q_off, H = 5, 96, 96, 4 * 96, 2
    q = dev(synth.normal(2200, "q", (1, Lq, H, 128)), "bf16")
    do = dev(synth.normal(2200, "do", (1, Lq, H, 128)), "bf16")
    k = [dev(synth.normal(2200, "k", (1, S, H, 128), shard=j), "bf16") for j in range(n)]
    v = [dev(synth.normal(2200, "v", (1, S, H, 128), shard=j), "bf16") for j in range(n)]
    order = [4, 3, 2, 1, 0]
    o, _, lse = path.ring_forward(q, k, v, order, S, q_off)
    a = path.ring_backward(q, k, v, o, lse, do, order, S, q_off)
    b = path.ring_backward(q, k, v, o, lse, do, order[::-1], S, q_off)
    torch.cuda.synchronize()
    assert rel_fro(host(a[0]), host(b[0])) <= 1e-5
    for j in range(n):
        assert rel_fro(host(a[1][j]), host(b[1][j])) <= 1e-5 and rel_fro(host(a[2][j]), host(b[2][j])) <= 1e-5
    # the accumulators are added to, not overwritten
    dq2 = a[0].clone()
    path.ring_backward(q, k, v, o, lse, do, order, S, q_off, dq_acc=dq2, dk_acc={}, dv_acc={})
    torch.cuda.synchronize()
    assert rel_fro(host(dq2), 2 * host(a[0])) <= 1e-6
    # a shard wholly in the causal future adds exactly zero when passed explicitly
    z = torch.zeros((1, S, H, 128), dtype=torch.float32, device="cuda")
    dq3 = a[0].clone()
    lwm.lwm_ring_step_bwd(q, k[0], v[0], o, lse, do, dq3, z, z.clone(), q_offset=0, k_offset=10 * S)
    torch.cuda.synchronize()
    assert torch.equal(dq3, a[0]) and not bool(z.any())


def test_ring_backward_reused_workspace_is_exact():
    """Later steps of a ring reuse the delta and rescaled lse the first step wrote into the workspace
    (path.ring_backward does): bit-identical accumulators to recomputing them at every step,
    including with packing, where the first shard visited is not the first in key order."""
    need_gpu()
    note("ring backward: reusing the first step's delta/lse workspace equals recomputing it")
    for segs in (False, True):
        n, S, Lq, q_off, H = 5, 96, 96, 4 * 96, 2
        seed = 2300 + int(segs)
        q = dev(synth.normal(seed, "q", (1, Lq, H, 128)), "bf16")
        do = dev(synth.normal(seed, "do", (1, Lq, H, 128)), "bf16")
        k = [dev(synth.normal(seed, "k", (1, S, H, 128), shard=j), "bf16") for j in range(n)]
        v = [dev(synth.normal(seed, "v", (1, S, H, 128), shard=j), "bf16") for j in range(n)]
        seg = synth.random_segment_ids(seed, 1, n * S, 70) if segs else None
        sq = None if seg is None else seg_dev(seg[:, q_off:q_off + Lq])
        sk = None if seg is None else [seg_dev(seg[:, j * S:(j + 1) * S]) for j in range(n)]
        order = [4, 3, 2, 1, 0]
        o, _, lse = path.ring_forward(q, k, v, order, S, q_off, seg_q=sq, seg_k_shards=sk)
        dq_r, dk_r, dv_r = path.ring_backward(q, k, v, o, lse, do, order, S, q_off, seg_q=sq, seg_k_shards=sk)
        dq_f = torch.zeros_like(dq_r)
        ws = torch.empty(lwm.lwm_blockattn_bwd_workspace_size(1, H, Lq, S, 128), dtype=torch.uint8, device="cuda")
        for j in order:
            dkj = torch.zeros((1, S, H, 128), dtype=torch.float32, device="cuda")
            dvj = torch.zeros_like(dkj)
            lwm.lwm_ring_step_bwd(q, k[j], v[j], o, lse, do, dq_f, dkj, dvj, seg_q=sq,
                                  seg_k=None if sk is None else sk[j], q_offset=q_off, k_offset=j * S, workspace=ws)
            torch.cuda.synchronize()
            assert torch.equal(dkj, dk_r[j]) and torch.equal(dvj, dv_r[j]), (segs, j)
        assert torch.equal(dq_f, dq_r), segs
    with pytest.raises(ValueError, match="reuse_workspace"):
        lwm.lwm_ring_step_bwd(q, k[0], v[0], o, lse, do, dq_f, dkj, dvj, q_offset=q_off, reuse_workspace=True)
