"""RoPE inside the attention calls (lwm_blockattn_fwd_rope / lwm_blockattn_bwd_rope).

The forward must equal, bit for bit, lwm_rope_apply on Q and K followed by lwm_blockattn_fwd (the
rotation is the same arithmetic, done in registers); the backward must match the oracle's
gradients w.r.t. the pre-RoPE Q and K, give dV bit for bit as lwm_blockattn_bwd does, and stay
within rounding of the separate route (which rounds dQ', dK' to bf16 before rotating them back).
"""
import numpy as np
import pytest
import torch

import oracle
from ring_causal_attention_amd import lwm, path, synth
from tests.gpu_utils import (BF16_MAX_ABS, BF16_MEAN_ABS, GRAD_REL_FRO, dev, errors, exact_host, host, need_gpu,
                             note, rel_fro, seg_dev)

pytestmark = pytest.mark.gpu


def separate_fwd(qd, kd, vd, theta, layout, segd, restart, q_offset, k_offset, qpo, kpo, causal):
    rs = segd if restart else None
    qr = lwm.lwm_rope_apply(qd, pos_offset=qpo, seg=rs, theta=theta, layout=layout)
    kr = lwm.lwm_rope_apply(kd, pos_offset=kpo, seg=rs, theta=theta, layout=layout)
    o, lse = lwm.lwm_blockattn_fwd(qr, kr, vd, segd, segd, q_offset, k_offset, causal)
    return o, lse, qr, kr


def fused_case(B, Lq, Lk, H, seed, theta=1e6, layout="half", seg=None, restart=False, q_offset=0, k_offset=0,
               qpo=0, kpo=0, causal=True, backward=True):
    note(f"fused rope B={B} Lq={Lq} Lk={Lk} H={H} theta={theta} layout={layout} seg={seg is not None} "
         f"restart={restart} offsets=({q_offset},{k_offset}) pos_offsets=({qpo},{kpo}) causal={causal}")
    q, k, v = (synth.normal(seed, t, (B, L, H, 128)) for t, L in (("q", Lq), ("k", Lk), ("v", Lk)))
    do = synth.normal(seed, "do", (B, Lq, H, 128))
    qd, kd, vd, dod = dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), dev(do, "bf16")
    segd = None if seg is None else seg_dev(seg)
    o, lse, qr, kr = lwm.lwm_blockattn_fwd_rope(qd, kd, vd, theta, segd, segd, q_offset, k_offset, causal,
                                                layout=layout, restart=restart, q_pos_offset=qpo, k_pos_offset=kpo)
    so, slse, sqr, skr = separate_fwd(qd, kd, vd, theta, layout, segd, restart, q_offset, k_offset, qpo, kpo, causal)
    torch.cuda.synchronize()
    assert torch.equal(qr, sqr) and torch.equal(kr, skr), "rotated operands differ from lwm_rope_apply"
    assert torch.equal(o, so), "fused forward differs from RoPE + forward"
    assert torch.equal(lse, slse)
    # against the oracle: RoPE of the exact inputs in float64, then the attention definition
    pos_q = oracle.positions(B, Lq, qpo, seg if restart else None)
    pos_k = oracle.positions(B, Lk, kpo, seg if restart else None)
    xq, xk, xv, xdo = (exact_host(x, "bf16") for x in (q, k, v, do))
    ro, rlse, rdq, rdk, rdv = oracle.training_step(xq, xk, xv, xdo, pos_q, pos_k, theta, layout, seg, seg,
                                                   q_offset, k_offset, causal)
    mx, mean = errors(host(o), ro)
    assert mx <= BF16_MAX_ABS and mean <= BF16_MEAN_ABS, (mx, mean)
    if not backward:
        return
    dq, dk, dv = lwm.lwm_blockattn_bwd_rope(qr, kr, vd, o, lse, dod, theta, segd, segd, q_offset, k_offset, causal,
                                            layout=layout, restart=restart, q_pos_offset=qpo, k_pos_offset=kpo)
    sdq, sdk, sdv = lwm.lwm_blockattn_bwd(sqr, skr, vd, so, slse, dod, segd, segd, q_offset, k_offset, causal)
    rs = segd if restart else None
    lwm.lwm_rope_apply(sdq, sdq, pos_offset=qpo, seg=rs, theta=theta, layout=layout, inverse=True)
    lwm.lwm_rope_apply(sdk, sdk, pos_offset=kpo, seg=rs, theta=theta, layout=layout, inverse=True)
    torch.cuda.synchronize()
    assert torch.equal(dv, sdv), "dV must not depend on where RoPE runs"
    for name, g, sg, r in (("dq", dq, sdq, rdq), ("dk", dk, sdk, rdk)):
        gg, ss = host(g), host(sg)
        assert np.all(np.isfinite(gg)), name
        if np.linalg.norm(r) == 0:
            assert np.max(np.abs(gg)) <= 1e-3, name
            continue
        assert rel_fro(gg, r) <= GRAD_REL_FRO, (name, rel_fro(gg, r))
        # one bf16 rounding (fused) against two (separate): a rounding-level difference only
        assert rel_fro(gg, ss) <= 6e-3, (name, rel_fro(gg, ss))


@pytest.mark.parametrize("L", [1, 63, 129, 300])
@pytest.mark.parametrize("layout", ["half", "interleaved"])
def test_causal(L, layout):
    need_gpu()
    fused_case(1, L, L, 2, 4000 + L, layout=layout)


def test_heads_batches_theta():
    need_gpu()
    fused_case(2, 200, 200, 4, 4101, theta=1e4)  # B*H multiple of 8: XCD-grouped order
    fused_case(1, 160, 160, 3, 4102, theta=5e7, qpo=655360, kpo=655360)


@pytest.mark.parametrize("layout", ["half", "interleaved"])
def test_packed_restart(layout):
    need_gpu()
    # short segments, one of length 1, and a wave of 32 rows that spans several segment starts
    seg = synth.segment_ids_from_lengths([40, 1, 7, 3, 90, 33, 126])
    fused_case(1, 300, 300, 2, 4200, layout=layout, seg=seg, restart=True)
    seg2 = synth.random_segment_ids(4201, 2, 333, 64)
    fused_case(2, 333, 333, 2, 4202, layout=layout, seg=seg2, restart=True)


def test_packed_without_restart():
    need_gpu()
    seg = synth.segment_ids_from_lengths([100, 156])
    fused_case(1, 256, 256, 2, 4300, seg=seg, restart=False)


def test_ring_like_offsets():
    need_gpu()
    # a query block after its keys: mask offsets and RoPE position offsets set independently
    fused_case(1, 150, 350, 2, 4400, q_offset=200, k_offset=0, qpo=200 + 655360, kpo=655360)
    fused_case(1, 129, 400, 2, 4401, q_offset=333, k_offset=17, qpo=1000, kpo=684)
    fused_case(1, 190, 77, 2, 4402, causal=False, qpo=5, kpo=9)


def test_strided_views():
    need_gpu()
    note("fused rope on views of a fused QKV buffer")
    B, L, H, theta = 1, 257, 2, 1e6
    x = synth.normal(4500, "q", (B, L, 3, H, 128))
    xd = dev(x, "bf16")
    qd, kd, vd = xd[:, :, 0], xd[:, :, 1], xd[:, :, 2]
    o, lse, qr, kr = lwm.lwm_blockattn_fwd_rope(qd, kd, vd, theta)
    so, slse, sqr, skr = separate_fwd(qd.contiguous(), kd.contiguous(), vd.contiguous(), theta, "half", None, False,
                                      0, 0, 0, 0, True)
    torch.cuda.synchronize()
    assert torch.equal(o, so) and torch.equal(lse, slse) and torch.equal(qr, sqr) and torch.equal(kr, skr)


def test_in_place_keys():
    need_gpu()
    note("fused rope with k_rot == k")
    q, k, v = (dev(synth.normal(4600, t, (1, 200, 2, 128)), "bf16") for t in ("q", "k", "v"))
    o, lse, qr, kr = lwm.lwm_blockattn_fwd_rope(q, k.clone(), v, 1e6)
    k2 = k.clone()
    o2, lse2, _, kr2 = lwm.lwm_blockattn_fwd_rope(q, k2, v, 1e6, k_rot=k2)
    torch.cuda.synchronize()
    assert kr2.data_ptr() == k2.data_ptr()
    assert torch.equal(kr2, kr) and torch.equal(o2, o) and torch.equal(lse2, lse)


def test_fused_training_step_full_size():
    """The L=32768, 32-head training step through the fused calls equals the separate route:
    O and lse bit for bit, dV bit for bit, dQ and dK within rounding; plus the exact gradient
    identities on the fused output."""
    need_gpu()
    note("fused training step L=32768 H=32 against the separate route")
    B, L, H, theta = 1, 32768, 32, 1e6
    q, k, v, do = (dev(synth.normal(1005, t, (B, L, H, 128)), "bf16") for t in ("q", "k", "v", "do"))
    bufs = path.TrainStepBuffers(q, k)
    o, lse, dq, dk, dv = (t.clone() for t in path.training_step_fused(q, k, v, do, theta, buffers=bufs))
    so, slse, sdq, sdk, sdv = path.training_step(q, k, v, do, theta, buffers=bufs)
    torch.cuda.synchronize()
    assert torch.equal(o, so) and torch.equal(lse, slse) and torch.equal(dv, sdv)
    for g, s in ((dq, sdq), (dk, sdk)):
        d = (g.float() - s.float()).norm() / s.float().norm()
        assert float(d) <= 6e-3, float(d)
    # sum_j dK'_j = 0 survives the inverse rotation per position only; check it on dV instead:
    # sum_j dV_j = sum_i dO_i (every row sees at least itself)
    sdv_sum = dv.float().sum(dim=1)
    sdo_sum = do.float().sum(dim=1)
    assert float((sdv_sum - sdo_sum).norm() / sdo_sum.norm()) <= 1e-2
