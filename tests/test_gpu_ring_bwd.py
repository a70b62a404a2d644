"""lwm_ring_step_bwd: KV shards visited backward around the ring, each adding its share of the
gradients, give the gradients of attention over all keys (oracle: the backward ring step summed
over shards, pinned against autograd through SDPA)."""
import numpy as np
import pytest
import torch

import oracle
from ring_causal_attention_amd import lwm, path, synth
from tests.gpu_utils import (BF16_MAX_ABS, BF16_MEAN_ABS, GRAD_REL_FRO, dev, errors, exact_host, host, need_gpu, note,
                             rel_fro, seg_dev)

pytestmark = pytest.mark.gpu


def ring_bwd_case(seed, n_shards, shard, Lq, q_off, H=2, segs=False, order=None):
    """GPU forward + backward ring against the oracle's per-shard contributions."""
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
    # the ring forward against attention over all keys
    ex_o, _ = oracle.attention_fwd(qe, ke, ve, seg_q, seg, q_off, 0, True)
    mx, mean = errors(host(o), ex_o)
    assert mx <= BF16_MAX_ABS and mean <= BF16_MEAN_ABS, ("o", mx, mean)
    # The backward step is defined on the forward's results: the oracle takes the O (bf16) and lse
    # that the kernels received.  With the exact O instead, a query that sees few keys turns the
    # bf16 rounding of O into a larger relative error of dP - delta (a cancellation) in the rows
    # of the shards it reaches, which is the forward's rounding, not the backward's.
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
    e = rel_fro(host(dq_acc), ref_dq)
    assert e <= GRAD_REL_FRO, ("dq", e)
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
