"""The five workloads at full size, run exactly as bench.py runs them, against the oracle.

Whole outputs are compared wherever the host can compute them in about a minute: every row and
head of the L = 32768 forward and of the packed L = 65536 forward, every row of two heads of the
1M-token ring share (sampled rows of the other six), four heads of the training step's O, lse and
gradients, and for the ring backward dQ on sampled query rows and dK / dV on sampled key rows of
two heads against the gradients of attention over all keys.  The oracle runs on the host cores in
parallel tasks (one BLAS thread each); these tests are marked ``slow``.
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch
from threadpoolctl import threadpool_limits

import oracle
from ring_causal_attention_amd import configs, lwm, path, synth, workloads
from ring_causal_attention_amd.synth import round_to_bf16
from tests.gpu_utils import (BF16_MAX_ABS, BF16_MEAN_ABS, FP32_MAX_ABS, GRAD_REL_FRO, LSE_BF16, errors, host,
                             need_gpu, note, rel_fro, report)

pytestmark = pytest.mark.gpu
W = configs.WORKLOADS


def exact(x, dtype):
    return (round_to_bf16(x) if dtype == "bf16" else x).astype(np.float64)


def host_threads() -> int:
    """Host cores this process may use, capped at 16 worker threads."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def pmap(fn, tasks, blas_threads=1):
    """fn over tasks in parallel threads, each with `blas_threads` BLAS threads."""
    workers = max(1, host_threads() // blas_threads)
    with threadpool_limits(blas_threads), ThreadPoolExecutor(max_workers=workers) as ex:
        return list(ex.map(fn, tasks))


class Stats:
    """Max-abs and mean-abs over a whole output assembled from parts."""

    def __init__(self):
        self.mx, self.total, self.n, self.lmx = 0.0, 0.0, 0, 0.0

    def add(self, got, ref, lse_got=None, lse_ref=None):
        d = np.abs(got - ref)
        self.mx = max(self.mx, float(d.max()))
        self.total += float(d.sum())
        self.n += d.size
        if lse_got is not None:
            self.lmx = max(self.lmx, float(np.max(np.abs(lse_got - lse_ref))))

    @property
    def mean(self):
        return self.total / max(self.n, 1)

    @staticmethod
    def merged(parts):
        st = Stats()
        for p in parts:
            st.mx, st.lmx = max(st.mx, p.mx), max(st.lmx, p.lmx)
            st.total, st.n = st.total + p.total, st.n + p.n
        return st


def sample_rows(L, extra=(), n_random=24, seed=0):
    base = {0, 1, 2, 63, 64, 127, 128, 129, L // 2, L - 2, L - 1}
    base |= {int(r) for r in extra if 0 <= r < L}
    base |= set(np.random.default_rng(seed).integers(0, L, n_random).tolist())
    return sorted(base)


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


@pytest.mark.slow
def test_llama7b_fwd_L32768_every_row_and_head():
    need_gpu()
    w = W["llama7b_fwd_L32768"]
    note(f"workload {w.name} (oracle on every row of every head)")
    h = workloads.host_inputs(w)
    d = workloads.device_inputs(h)
    o, lse, _, _ = path.attention_forward(d["q"], d["k"], d["v"], w.theta)
    torch.cuda.synchronize()
    # row 0 sees only key 0: O_0 = V_0 exactly
    assert torch.equal(o[:, 0].float(), d["v"][:, 0].float())
    got_o, got_l = host(o), host(lse)
    del d, o, lse
    pos = oracle.positions(w.B, w.Lq)

    def one(hh):
        sl = lambda x: exact(x[:, :, hh:hh + 1], "bf16")
        qr, kr = oracle.rope(sl(h["q"]), pos, w.theta), oracle.rope(sl(h["k"]), pos, w.theta)
        ro, rl = oracle.attention_fwd(qr, kr, sl(h["v"]), threads=1)
        st = Stats()
        st.add(got_o[:, :, hh:hh + 1], ro, got_l[:, hh:hh + 1], rl)
        return st

    st = Stats.merged(pmap(one, range(w.H)))
    assert st.n == got_o.size
    report(w.name, rows="all", heads=w.H, o_max_abs=st.mx, o_mean_abs=st.mean, lse_max_abs=st.lmx)
    assert st.mx <= BF16_MAX_ABS and st.mean <= BF16_MEAN_ABS, (st.mx, st.mean)
    assert st.lmx <= LSE_BF16, st.lmx


@pytest.mark.slow
def test_packed_L65536_every_row_and_head():
    need_gpu()
    w = W["packed_L65536"]
    note(f"workload {w.name} (oracle on every row of every head)")
    h = workloads.host_inputs(w)
    d = workloads.device_inputs(h)
    o, lse, _, _ = path.attention_forward(d["q"], d["k"], d["v"], w.theta, seg=d["seg"])
    torch.cuda.synchronize()
    lens = w.segment_lengths()
    starts = np.cumsum([0] + lens[:-1])
    # every segment start returns its own V row bit for bit
    assert torch.equal(o[:, starts].float(), d["v"][:, starts].float())
    got_o, got_l = host(o), host(lse)
    del d, o, lse
    seg = h["seg"]
    pos = oracle.positions(w.B, w.Lq, 0, seg)

    # Keys outside a query's segment are invisible, so the oracle over all keys restricted to the
    # rows of one segment equals the oracle over that segment's keys (same ids, offsets, positions).
    def one(task):
        hh, a, b = task
        sl = lambda x: exact(x[:, a:b, hh:hh + 1], "bf16")
        qr = oracle.rope(sl(h["q"]), pos[:, a:b], w.theta)
        kr = oracle.rope(sl(h["k"]), pos[:, a:b], w.theta)
        ro, rl = oracle.attention_fwd(qr, kr, sl(h["v"]), seg[:, a:b], seg[:, a:b], a, a, True, threads=1)
        st = Stats()
        st.add(got_o[:, a:b, hh:hh + 1], ro, got_l[:, hh:hh + 1, a:b], rl)
        return st

    tasks = [(hh, int(a), int(a + n)) for hh in range(w.H) for a, n in zip(starts, lens)]
    st = Stats.merged(pmap(one, sorted(tasks, key=lambda t: t[1] - t[2])))
    assert st.n == got_o.size
    report(w.name, rows="all", heads=w.H, segments=len(lens), o_max_abs=st.mx, o_mean_abs=st.mean,
           lse_max_abs=st.lmx)
    assert st.mx <= BF16_MAX_ABS and st.mean <= BF16_MEAN_ABS, (st.mx, st.mean)
    assert st.lmx <= LSE_BF16, st.lmx


def test_packed_L65536_training_step_one_head():
    need_gpu()
    w = W["packed_L65536"]
    note(f"workload {w.name} training step")
    h = workloads.host_inputs(w)
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


# ------------------------------------------------------------------ the 1M-token ring share
RING_HEADS = [0, 5]


@pytest.fixture(scope="module")
def ring_share():
    """Inputs of the ring share, the GPU's ring forward, and the oracle's O and lse over all keys
    for every query row of RING_HEADS (float64), shared by the forward and backward checks."""
    need_gpu()
    w = W["ring_share_1M"]
    h = workloads.host_inputs(w)
    S, r = w.Lq, w.ring_index
    k_all = np.concatenate([h["k_shards"][j] for j in range(r + 1)], axis=1)
    v_all = np.concatenate([h["v_shards"][j] for j in range(r + 1)], axis=1)
    pos_q = oracle.positions(w.B, S, w.q_offset)
    pos_k = oracle.positions(w.B, k_all.shape[1])
    # per head, contiguous: the oracle reads one head's keys as a [L, D] view without copying
    qr = [oracle.rope(exact(h["q"][:, :, hh:hh + 1], "bf16"), pos_q, w.theta) for hh in RING_HEADS]
    kr = [oracle.rope(exact(k_all[:, :, hh:hh + 1], "bf16"), pos_k, w.theta) for hh in RING_HEADS]
    vr = [exact(v_all[:, :, hh:hh + 1], "bf16") for hh in RING_HEADS]
    chunk = 512

    def one(task):
        n, r0 = task
        rows = np.arange(r0, min(S, r0 + chunk))
        o, l = oracle.attention_fwd(qr[n], kr[n], vr[n], None, None, w.q_offset, 0, True, rows=rows, row_block=64,
                                    threads=1)
        return task, o, l

    ex_o = np.zeros((w.B, S, len(RING_HEADS), w.D))
    ex_l = np.zeros((w.B, len(RING_HEADS), S))
    for (n, r0), o, l in pmap(one, [(n, r0) for n in range(len(RING_HEADS)) for r0 in range(0, S, chunk)]):
        ex_o[:, r0:r0 + o.shape[1], n] = o[:, :, 0]
        ex_l[:, n, r0:r0 + o.shape[1]] = l[:, 0]
    return dict(w=w, h=h, k_all=k_all, v_all=v_all, pos_q=pos_q, pos_k=pos_k, qr=qr, kr=kr, vr=vr, ex_o=ex_o,
                ex_l=ex_l)


def ring_device_forward(w, h):
    d = workloads.device_inputs(h)
    qr = lwm.lwm_rope_apply(d["q"], pos_offset=w.q_offset, theta=w.theta)
    kr = {j: lwm.lwm_rope_apply(x, pos_offset=j * w.Lq, theta=w.theta) for j, x in d["k_shards"].items()}
    o, _, lse = path.ring_forward(qr, kr, d["v_shards"], w.ring_order(), w.Lq, w.q_offset)
    return d, qr, kr, o, lse


@pytest.mark.slow
def test_ring_share_1M_every_row_of_two_heads(ring_share):
    rs = ring_share
    w, h = rs["w"], rs["h"]
    note(f"workload {w.name} (every row of heads {RING_HEADS}, sampled rows of the others)")
    d, qr, kr, o, lse = ring_device_forward(w, h)
    torch.cuda.synchronize()
    got_o, got_l = host(o), host(lse)
    del d, qr, kr, o, lse
    st = Stats()
    st.add(got_o[:, :, RING_HEADS], rs["ex_o"], got_l[:, RING_HEADS], rs["ex_l"])
    report(w.name, rows="all", heads=len(RING_HEADS), o_max_abs=st.mx, o_mean_abs=st.mean, lse_max_abs=st.lmx)
    assert st.mx <= BF16_MAX_ABS and st.mean <= BF16_MEAN_ABS, (st.mx, st.mean)
    assert st.lmx <= LSE_BF16, st.lmx
    # the other heads on sampled rows
    others = [x for x in range(w.H) if x not in RING_HEADS]
    rows = sample_rows(w.Lq, n_random=12, seed=4)

    def one(hh):
        q_h = oracle.rope(exact(h["q"][:, :, hh:hh + 1], "bf16"), rs["pos_q"], w.theta)
        k_h = oracle.rope(exact(rs["k_all"][:, :, hh:hh + 1], "bf16"), rs["pos_k"], w.theta)
        ro, rl = oracle.attention_fwd(q_h, k_h, exact(rs["v_all"][:, :, hh:hh + 1], "bf16"), None, None, w.q_offset,
                                      0, True, rows=rows, row_block=1, threads=1)
        st = Stats()
        st.add(got_o[:, rows][:, :, hh:hh + 1], ro, got_l[:, hh:hh + 1][:, :, rows], rl)
        return st

    st2 = Stats.merged(pmap(one, others))
    report(w.name + "_other_heads", rows=len(rows), heads=len(others), o_max_abs=st2.mx, o_mean_abs=st2.mean,
           lse_max_abs=st2.lmx)
    assert st2.mx <= BF16_MAX_ABS and st2.mean <= BF16_MEAN_ABS, (st2.mx, st2.mean)
    assert st2.lmx <= LSE_BF16, st2.lmx


@pytest.mark.slow
def test_ring_share_1M_backward(ring_share):
    rs = ring_share
    w, h = rs["w"], rs["h"]
    S, r = w.Lq, w.ring_index
    note(f"workload {w.name} backward (dQ rows and dK / dV key rows of heads {RING_HEADS})")
    d, qr, kr, o, lse = ring_device_forward(w, h)
    dq_acc, dk_acc, dv_acc = path.ring_backward(qr, kr, d["v_shards"], o, lse, d["do"], w.ring_order(), S, w.q_offset)
    torch.cuda.synchronize()
    assert sorted(dk_acc) == list(range(r + 1))
    # at any size: rows of P sum to one over all keys, so sum over every key of dV = sum_i dO_i
    sdv = sum(x.sum(dim=1) for x in dv_acc.values()).cpu().numpy()
    sdo = exact(h["do"], "bf16").sum(axis=1)
    assert np.linalg.norm(sdv - sdo) <= 1e-2 * np.linalg.norm(sdo)
    hs = RING_HEADS
    doe = [exact(h["do"][:, :, hh:hh + 1], "bf16") for hh in hs]
    ex_o = [np.ascontiguousarray(rs["ex_o"][:, :, n:n + 1]) for n in range(len(hs))]
    ex_l = [np.ascontiguousarray(rs["ex_l"][:, n:n + 1]) for n in range(len(hs))]
    qr_h, kr_h, vr_h = rs["qr"], rs["kr"], rs["vr"]
    # dQ of sampled query rows: exact gradients of attention over all keys (oracle O and lse)
    qrows = sample_rows(S, n_random=10, seed=5)

    def dq_row(task):
        n, row = task
        sl = slice(row, row + 1)
        g, _, _ = oracle.ring_step_bwd(qr_h[n][:, sl], kr_h[n], vr_h[n], ex_o[n][:, sl], ex_l[n][:, :, sl],
                                       doe[n][:, sl], None, None, w.q_offset + row, 0, True, row_block=1, threads=1)
        return task, g[:, 0, 0]

    ref_dq = np.zeros((w.B, len(qrows), len(hs), w.D))
    for (n, row), g in pmap(dq_row, [(n, row) for n in range(len(hs)) for row in qrows]):
        ref_dq[:, qrows.index(row), n] = g
    got_dq = host(dq_acc[:, qrows][:, :, hs])
    e_dq = rel_fro(got_dq, ref_dq)
    # dK and dV of sampled key rows (every shard's first and last key, the diagonal shard's
    # edges, random keys): a one-key shard's share under the exact O and lse of all keys is the
    # whole gradient of that key
    Lk = (r + 1) * S
    krows = sorted({j * S for j in range(r + 1)} | {j * S + S - 1 for j in range(r + 1)}
                   | {r * S + 1, r * S + S // 2, Lk - 2}
                   | set(np.random.default_rng(6).integers(0, Lk, 16).tolist()))

    def dkv_row(task):
        n, g = task
        sl = slice(g, g + 1)
        _, dk1, dv1 = oracle.ring_step_bwd(qr_h[n], kr_h[n][:, sl], vr_h[n][:, sl], ex_o[n], ex_l[n], doe[n], None,
                                           None, w.q_offset, g, True, threads=1)
        return task, dk1[:, 0, 0], dv1[:, 0, 0]

    ref_dk = np.zeros((w.B, len(krows), len(hs), w.D))
    ref_dv = np.zeros_like(ref_dk)
    for (n, g), a, b in pmap(dkv_row, [(n, g) for n in range(len(hs)) for g in krows]):
        ref_dk[:, krows.index(g), n] = a
        ref_dv[:, krows.index(g), n] = b
    got_dk = np.stack([host(dk_acc[g // S][:, g % S][:, hs]) for g in krows], axis=1)
    got_dv = np.stack([host(dv_acc[g // S][:, g % S][:, hs]) for g in krows], axis=1)
    e_dk, e_dv = rel_fro(got_dk, ref_dk), rel_fro(got_dv, ref_dv)
    report(w.name + "_backward", dq_rows=len(qrows), key_rows=len(krows), heads=len(hs), dq_rel_fro=e_dq,
           dk_rel_fro=e_dk, dv_rel_fro=e_dv, sum_dv_vs_sum_do=float(np.linalg.norm(sdv - sdo) / np.linalg.norm(sdo)))
    assert e_dq <= GRAD_REL_FRO, e_dq
    assert e_dk <= GRAD_REL_FRO, e_dk
    assert e_dv <= GRAD_REL_FRO, e_dv


# ------------------------------------------------------------------ the L = 32768 training step
TRAIN_HEADS = [0, 11, 20, 31]


@pytest.mark.slow
def test_train_step_L32768_four_heads():
    need_gpu()
    w = W["train_step_L32768"]
    note(f"workload {w.name} (O, lse and gradients of heads {TRAIN_HEADS}, every row)")
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
    hs = TRAIN_HEADS
    got = {name: host(t[:, :, hs]) for name, t in (("o", o), ("dq", dq), ("dk", dk), ("dv", dv))}
    got_l = host(lse[:, hs])
    del d, o, lse, dq, dk, dv
    pos = oracle.positions(w.B, w.Lq)

    def one(n):
        hh = hs[n]
        sl = lambda x: exact(x[:, :, hh:hh + 1], "bf16")
        return n, oracle.training_step(sl(h["q"]), sl(h["k"]), sl(h["v"]), sl(h["do"]), pos, pos, w.theta, "half",
                                       threads=1)

    ref = {name: np.zeros_like(got[name]) for name in got}
    ref_l = np.zeros_like(got_l)
    for n, (ro, rl, rdq, rdk, rdv) in pmap(one, range(len(hs)), blas_threads=max(1, host_threads() // len(hs))):
        for name, x in (("o", ro), ("dq", rdq), ("dk", rdk), ("dv", rdv)):
            ref[name][:, :, n] = x[:, :, 0]
        ref_l[:, n] = rl[:, 0]
    mx, mean = errors(got["o"], ref["o"])
    lmx = float(np.max(np.abs(got_l - ref_l)))
    errs = {name: rel_fro(got[name], ref[name]) for name in ("dq", "dk", "dv")}
    per_head = {f"{name}_h{hh}": rel_fro(got[name][:, :, n], ref[name][:, :, n]) for n, hh in enumerate(hs)
                for name in ("dq", "dk", "dv")}
    report(w.name, heads=len(hs), o_max_abs=mx, o_mean_abs=mean, lse_max_abs=lmx,
           **{f"{k}_rel_fro": v for k, v in errs.items()},
           worst_head_rel_fro=max(per_head.values()),
           sum_dv_vs_sum_do=float(np.linalg.norm(sdv - sdo) / np.linalg.norm(sdo)))
    assert mx <= BF16_MAX_ABS and mean <= BF16_MEAN_ABS, (mx, mean)
    assert lmx <= LSE_BF16, lmx
    for name, e in list(errs.items()) + list(per_head.items()):
        assert e <= GRAD_REL_FRO, (name, e)
