"""The five workloads at full size, run exactly as bench.py runs them, against the oracle.

Full-size outputs are checked on sampled rows the oracle computes one by one (every row of the
small fp32 workload; one full head for the training step's gradients), plus properties that hold
at any size.
"""
import numpy as np
import pytest
import torch

import oracle
from ring_causal_attention_amd import configs, lwm, path, workloads
from ring_causal_attention_amd.synth import round_to_bf16
from tests.gpu_utils import (BF16_MAX_ABS, BF16_MEAN_ABS, FP32_MAX_ABS, GRAD_REL_FRO, LSE_BF16, errors, host,
                             need_gpu, note, rel_fro, report)

pytestmark = pytest.mark.gpu
W = configs.WORKLOADS


def exact(x, dtype):
    return (round_to_bf16(x) if dtype == "bf16" else x).astype(np.float64)


def sample_rows(L, extra=(), n_random=24, seed=0):
    base = {0, 1, 2, 63, 64, 127, 128, 129, L // 2, L - 2, L - 1}
    base |= {int(r) for r in extra if 0 <= r < L}
    base |= set(np.random.default_rng(seed).integers(0, L, n_random).tolist())
    return sorted(base)


def oracle_rows(q, k, v, rows, theta, dtype, pos_q, pos_k, seg=None, q_offset=0, k_offset=0, heads=None):
    """Oracle O, lse for the chosen query rows (RoPE and attention in float64), one row at a time."""
    hs = slice(None) if heads is None else list(heads)
    maxlim = min(k.shape[1], q_offset + max(rows) - k_offset + 1)
    kr_all = oracle.rope(exact(k[:, :maxlim][:, :, hs], dtype), pos_k[:, :maxlim], theta)
    vr_all = exact(v[:, :maxlim][:, :, hs], dtype)
    o_rows, l_rows = [], []
    for r in rows:
        lim = min(k.shape[1], q_offset + r - k_offset + 1)
        qr = oracle.rope(exact(q[:, r:r + 1][:, :, hs], dtype), pos_q[:, r:r + 1], theta)
        sq = None if seg is None else seg[:, r:r + 1]
        sk = None if seg is None else seg[:, :lim]
        o, l = oracle.attention_fwd(qr, kr_all[:, :lim], vr_all[:, :lim], sq, sk, q_offset + r, k_offset, True)
        o_rows.append(o[:, 0])
        l_rows.append(l[:, :, 0])
    return np.stack(o_rows, 1), np.stack(l_rows, 2)


def check_rows(o_dev, lse_dev, ref_o, ref_l, rows, dtype, heads=None):
    hs = slice(None) if heads is None else list(heads)
    got = host(o_dev[:, rows][:, :, hs])
    gl = host(lse_dev[:, hs][:, :, rows]) if lse_dev is not None else None
    mx, mean = errors(got, ref_o)
    if dtype == "bf16":
        assert mx <= BF16_MAX_ABS and mean <= BF16_MEAN_ABS, (mx, mean)
    else:
        assert mx <= FP32_MAX_ABS, mx
    lmx = float(np.max(np.abs(gl - ref_l))) if gl is not None else None
    if gl is not None:
        assert lmx <= (LSE_BF16 if dtype == "bf16" else 1e-5)
    return mx, mean, lmx


def test_causal_fp32_L1024_full():
    need_gpu()
    w = W["causal_fp32_L1024"]
    note(f"workload {w.name}")
    h = workloads.host_inputs(w)
    d = workloads.device_inputs(h)
    o, lse, _, _ = path.attention_forward(d["q"], d["k"], d["v"], w.theta)
    torch.cuda.synchronize()
    pos = oracle.positions(w.B, w.Lq)
    qr, kr = oracle.rope(exact(h["q"], "fp32"), pos, w.theta), oracle.rope(exact(h["k"], "fp32"), pos, w.theta)
    ro, rl = oracle.attention_fwd(qr, kr, exact(h["v"], "fp32"))
    mx, mean = errors(host(o), ro)
    lmx = float(np.max(np.abs(host(lse) - rl)))
    report(w.name, rows="all", o_max_abs=mx, o_mean_abs=mean, lse_max_abs=lmx)
    assert mx <= FP32_MAX_ABS, mx
    assert lmx <= 1e-5


def test_llama7b_fwd_L32768_sampled():
    need_gpu()
    w = W["llama7b_fwd_L32768"]
    note(f"workload {w.name}")
    h = workloads.host_inputs(w)
    d = workloads.device_inputs(h)
    o, lse, _, _ = path.attention_forward(d["q"], d["k"], d["v"], w.theta)
    torch.cuda.synchronize()
    assert not bool(torch.isnan(o).any())
    rows = sample_rows(w.Lq, seed=2)
    pos = oracle.positions(w.B, w.Lq)
    ro, rl = oracle_rows(h["q"], h["k"], h["v"], rows, w.theta, "bf16", pos, pos)
    mx, mean, lmx = check_rows(o, lse, ro, rl, rows, "bf16")
    report(w.name, rows=len(rows), o_max_abs=mx, o_mean_abs=mean, lse_max_abs=lmx)
    # row 0 sees only key 0: O_0 = V_0 exactly
    assert torch.equal(o[:, 0].float(), d["v"][:, 0].float())


def test_packed_L65536_sampled():
    need_gpu()
    w = W["packed_L65536"]
    note(f"workload {w.name}")
    h = workloads.host_inputs(w)
    d = workloads.device_inputs(h)
    o, lse, _, _ = path.attention_forward(d["q"], d["k"], d["v"], w.theta, seg=d["seg"])
    torch.cuda.synchronize()
    lens = w.segment_lengths()
    starts = np.cumsum([0] + lens[:-1])
    ends = starts + np.array(lens) - 1
    rows = sample_rows(w.Lq, extra=list(starts) + list(ends), seed=3)
    pos = oracle.positions(w.B, w.Lq, 0, h["seg"])
    ro, rl = oracle_rows(h["q"], h["k"], h["v"], rows, w.theta, "bf16", pos, pos, seg=h["seg"])
    mx, mean, lmx = check_rows(o, lse, ro, rl, rows, "bf16")
    report(w.name, rows=len(rows), o_max_abs=mx, o_mean_abs=mean, lse_max_abs=lmx)
    # every segment start returns its own V row bit for bit
    assert torch.equal(o[:, starts].float(), d["v"][:, starts].float())


def test_packed_L65536_training_step_one_head():
    need_gpu()
    w = W["packed_L65536"]
    note(f"workload {w.name} training step")
    h = workloads.host_inputs(w)
    from ring_causal_attention_amd import synth
    do_h = synth.normal(w.seed, "do", (w.B, w.Lq, w.H, w.D))
    d = workloads.device_inputs(h)
    o, lse, dq, dk, dv = path.training_step(d["q"], d["k"], d["v"], workloads.to_device(do_h, w.dtype), w.theta,
                                            seg=d["seg"])
    torch.cuda.synchronize()
    for t in (dq, dk, dv):
        assert not bool(torch.isnan(t).any())
    # every row sees at least itself: sum over keys of dV = sum over queries of dO, all heads
    sdv = dv.float().sum(dim=1).cpu().numpy()
    sdo = exact(do_h, "bf16").sum(axis=1)
    assert np.linalg.norm(sdv - sdo) <= 1e-2 * np.linalg.norm(sdo)
    # one full head against the oracle, segment by segment: a packed segment is exactly an
    # unpacked causal sequence of its own with positions from 0 (an oracle pin checks this)
    hh = 11
    sl = lambda x, a, b: exact(x[:, a:b, hh:hh + 1], "bf16")
    ro, rdq, rdk, rdv = (np.zeros((w.B, w.Lq, 1, w.D)) for _ in range(4))
    start = 0
    for n in w.segment_lengths():
        a, b = start, start + n
        pos = oracle.positions(w.B, n)
        o_s, _, dq_s, dk_s, dv_s = oracle.training_step(sl(h["q"], a, b), sl(h["k"], a, b), sl(h["v"], a, b),
                                                        sl(do_h, a, b), pos, pos, w.theta, "half")
        ro[:, a:b], rdq[:, a:b], rdk[:, a:b], rdv[:, a:b] = o_s, dq_s, dk_s, dv_s
        start = b
    assert start == w.Lq
    mx, mean = errors(host(o[:, :, hh:hh + 1]), ro)
    errs = {name: rel_fro(host(g[:, :, hh:hh + 1]), ref) for name, g, ref in (("dq", dq, rdq), ("dk", dk, rdk),
                                                                            ("dv", dv, rdv))}
    report(w.name + "_train", head=hh, o_max_abs=mx, o_mean_abs=mean, **{f"{k}_rel_fro": v for k, v in errs.items()},
           sum_dv_vs_sum_do=float(np.linalg.norm(sdv - sdo) / np.linalg.norm(sdo)))
    assert mx <= BF16_MAX_ABS and mean <= BF16_MEAN_ABS, (mx, mean)
    for name, e in errs.items():
        assert e <= GRAD_REL_FRO, (name, e)


def test_ring_share_1M_sampled():
    need_gpu()
    w = W["ring_share_1M"]
    note(f"workload {w.name}")
    h = workloads.host_inputs(w)
    d = workloads.device_inputs(h)
    S, r = w.Lq, w.ring_index
    qr = lwm.lwm_rope_apply(d["q"], pos_offset=w.q_offset, theta=w.theta)
    kr = {j: lwm.lwm_rope_apply(x, pos_offset=j * S, theta=w.theta) for j, x in d["k_shards"].items()}
    o, o_acc, lse = path.ring_forward(qr, kr, d["v_shards"], w.ring_order(), S, w.q_offset)
    torch.cuda.synchronize()
    heads = [0, 5]
    rows = sample_rows(S, n_random=12, seed=4)
    k_all = np.concatenate([h["k_shards"][j] for j in range(r + 1)], axis=1)
    v_all = np.concatenate([h["v_shards"][j] for j in range(r + 1)], axis=1)
    pos_q = oracle.positions(w.B, S, w.q_offset)
    pos_k = oracle.positions(w.B, k_all.shape[1])
    ro, rl = oracle_rows(h["q"], k_all, v_all, rows, w.theta, "bf16", pos_q, pos_k, q_offset=w.q_offset,
                         heads=heads)
    mx, mean, lmx = check_rows(o, lse, ro, rl, rows, "bf16", heads=heads)
    report(w.name, rows=len(rows), heads=len(heads), o_max_abs=mx, o_mean_abs=mean, lse_max_abs=lmx)


def test_ring_share_1M_backward_sampled():
    need_gpu()
    w = W["ring_share_1M"]
    note(f"workload {w.name} backward")
    h = workloads.host_inputs(w)
    d = workloads.device_inputs(h)
    S, r = w.Lq, w.ring_index
    qr = lwm.lwm_rope_apply(d["q"], pos_offset=w.q_offset, theta=w.theta)
    kr = {j: lwm.lwm_rope_apply(x, pos_offset=j * S, theta=w.theta) for j, x in d["k_shards"].items()}
    o, _, lse = path.ring_forward(qr, kr, d["v_shards"], w.ring_order(), S, w.q_offset)
    dq_acc, dk_acc, dv_acc = path.ring_backward(qr, kr, d["v_shards"], o, lse, d["do"], w.ring_order(), S, w.q_offset)
    torch.cuda.synchronize()
    assert sorted(dk_acc) == list(range(r + 1))
    # at any size: rows of P sum to one over all keys, so sum over every key of dV = sum_i dO_i
    sdv = sum(x.sum(dim=1) for x in dv_acc.values()).cpu().numpy()
    sdo = exact(h["do"], "bf16").sum(axis=1)
    assert np.linalg.norm(sdv - sdo) <= 1e-2 * np.linalg.norm(sdo)
    # sampled query rows of dQ (w.r.t. the rotated Q) against the oracle's ring steps summed
    heads = [0, 5]
    rows = sample_rows(S, n_random=3, seed=5)[::3]
    k_all = np.concatenate([h["k_shards"][j] for j in range(r + 1)], axis=1)
    v_all = np.concatenate([h["v_shards"][j] for j in range(r + 1)], axis=1)
    pos_q = oracle.positions(w.B, S, w.q_offset)
    pos_k = oracle.positions(w.B, k_all.shape[1])
    ro, rl = oracle_rows(h["q"], k_all, v_all, rows, w.theta, "bf16", pos_q, pos_k, q_offset=w.q_offset,
                         heads=heads)
    kr_all = oracle.rope(exact(k_all[:, :, heads], "bf16"), pos_k, w.theta)
    vr_all = exact(v_all[:, :, heads], "bf16")
    ref = np.zeros((w.B, len(rows), len(heads), w.D))
    for n, row in enumerate(rows):
        qrow = oracle.rope(exact(h["q"][:, row:row + 1][:, :, heads], "bf16"), pos_q[:, row:row + 1], w.theta)
        dorow = exact(h["do"][:, row:row + 1][:, :, heads], "bf16")
        for j in range(r + 1):
            sl = slice(j * S, (j + 1) * S)
            dqj, _, _ = oracle.ring_step_bwd(qrow, kr_all[:, sl], vr_all[:, sl], ro[:, n:n + 1],
                                             rl[:, :, n:n + 1], dorow, None, None, w.q_offset + row, j * S, True)
            ref[:, n] += dqj[:, 0]
    got = host(dq_acc[:, rows][:, :, heads])
    report(w.name + "_backward", rows=len(rows), heads=len(heads), dq_rel_fro=rel_fro(got, ref),
           sum_dv_vs_sum_do=float(np.linalg.norm(sdv - sdo) / np.linalg.norm(sdo)))
    assert rel_fro(got, ref) <= GRAD_REL_FRO, rel_fro(got, ref)


def test_train_step_L32768_one_head():
    need_gpu()
    w = W["train_step_L32768"]
    note(f"workload {w.name}")
    h = workloads.host_inputs(w)
    d = workloads.device_inputs(h)
    o, lse, dq, dk, dv = path.training_step(d["q"], d["k"], d["v"], d["do"], w.theta)
    torch.cuda.synchronize()
    for t in (dq, dk, dv):
        assert not bool(torch.isnan(t).any())
    # exact identities of the gradient at full size, all heads: sum_j dV_j = sum_i dO_i
    sdv = dv.float().sum(dim=1).cpu().numpy()
    sdo = exact(h["do"], "bf16").sum(axis=1)
    assert np.linalg.norm(sdv - sdo) <= 1e-2 * np.linalg.norm(sdo)
    # one full head against the oracle's training step (forward, backward, inverse RoPE)
    hh = 7
    pos = oracle.positions(w.B, w.Lq)
    sl = lambda x: exact(x[:, :, hh:hh + 1], "bf16")
    ro, rl, rdq, rdk, rdv = oracle.training_step(sl(h["q"]), sl(h["k"]), sl(h["v"]), sl(h["do"]), pos, pos,
                                                 w.theta, "half")
    mx, mean = errors(host(o[:, :, hh:hh + 1]), ro)
    lmx = float(np.max(np.abs(host(lse[:, hh:hh + 1]) - rl)))
    errs = {name: rel_fro(host(g[:, :, hh:hh + 1]), ref) for name, g, ref in (("dq", dq, rdq), ("dk", dk, rdk),
                                                                            ("dv", dv, rdv))}
    report(w.name, head=hh, o_max_abs=mx, o_mean_abs=mean, lse_max_abs=lmx,
           **{f"{k}_rel_fro": v for k, v in errs.items()},
           sum_dv_vs_sum_do=float(np.linalg.norm(sdv - sdo) / np.linalg.norm(sdo)))
    assert mx <= BF16_MAX_ABS and mean <= BF16_MEAN_ABS, (mx, mean)
    for name, e in errs.items():
        assert e <= GRAD_REL_FRO, (name, e)
