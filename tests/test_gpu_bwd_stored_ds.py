"""The stored-dS backward (the dK/dV kernel also writes dS^T, dQ = scale dS K is formed from it)
against the recomputing backward on the same inputs, and against the oracle.

Both paths form the same bf16 dS from the same float32 arithmetic and add dQ up over the keys in
the same order, so their results agree bit for bit.  The workspace is filled with 0xFF bytes (NaN
as bf16) before each stored-dS call: pairs the dK/dV kernel never reaches keep that garbage, and
the dQ kernel must clear every invisible pair before its product.
"""
import numpy as np
import pytest
import torch

import oracle
from ring_causal_attention_amd import lwm, path, synth
from tests.gpu_utils import GRAD_REL_FRO, dev, exact_host, host, need_gpu, note, rel_fro, report, seg_dev, seg_pair_dev

pytestmark = pytest.mark.gpu


def poisoned_workspace(B, H, Lq, Lk, ds_heads, q_offset=0, k_offset=0, causal=True):
    ws = lwm.bwd_workspace(B, H, Lq, Lk, 128, "cuda", ds_heads, q_offset, k_offset, causal)
    ws.fill_(255)
    return ws


def stored_launches(fn):
    """Run fn with the library's launch timing on; return how many dQ-from-dS launches it made (the
    stored-dS path must really run where a test means it to)."""
    lwm.lwm_profile_reset()
    lwm.lwm_profile_enable(True)
    try:
        out = fn()
        torch.cuda.synchronize()
        prof = lwm.lwm_profile_read()
    finally:
        lwm.lwm_profile_enable(False)
    return out, prof.get("bwd_dq_ds", (0.0, 0))[1]


def inputs(B, Lq, Lk, H, seed, segs):
    q, k, v = (synth.normal(seed, t, (B, L, H, 128)) for t, L in (("q", Lq), ("k", Lk), ("v", Lk)))
    do = synth.normal(seed, "do", (B, Lq, H, 128))
    sq = sk = None
    if segs:
        seg = synth.random_segment_ids(seed, B, max(Lq, Lk), 150)
        sq, sk = seg[:, :Lq], seg[:, :Lk]
    return q, k, v, do, sq, sk


def stored_vs_recomputed(B, Lq, Lk, H, seed, segs=False, q_offset=0, k_offset=0, causal=True, heads=(None,)):
    need_gpu()
    note(f"stored dS B={B} Lq={Lq} Lk={Lk} H={H} segs={segs} q_off={q_offset} k_off={k_offset} causal={causal} "
         f"heads={heads}")
    q, k, v, do, sq, sk = inputs(B, Lq, Lk, H, seed, segs)
    qd, kd, vd, dod = dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), dev(do, "bf16")
    sqd, skd = seg_pair_dev(sq, sk, seed)
    o, lse = lwm.lwm_blockattn_fwd(qd, kd, vd, sqd, skd, q_offset, k_offset, causal)
    ref = lwm.lwm_blockattn_bwd(qd, kd, vd, o, lse, dod, sqd, skd, q_offset, k_offset, causal,
                                workspace=lwm.bwd_workspace(B, H, Lq, Lk, 128, "cuda", 0))
    got = None
    for g in heads:
        per_pass = lwm.default_ds_heads(B, H, Lq, Lk, 128, q_offset=q_offset, k_offset=k_offset,
                                        causal=causal) if g is None else g
        assert per_pass > 0
        ws = poisoned_workspace(B, H, Lq, Lk, g, q_offset, k_offset, causal)
        got, n = stored_launches(lambda: lwm.lwm_blockattn_bwd(qd, kd, vd, o, lse, dod, sqd, skd, q_offset, k_offset,
                                                               causal, workspace=ws))
        assert n == -(-(B * H) // per_pass), (n, per_pass)
        for name, a, r in zip(("dq", "dk", "dv"), got, ref):
            assert torch.equal(a, r), (name, g, float((a.float() - r.float()).abs().max()))
    rdq, rdk, rdv = oracle.attention_bwd(exact_host(q, "bf16"), exact_host(k, "bf16"), exact_host(v, "bf16"),
                                         exact_host(do, "bf16"), sq, sk, q_offset, k_offset, causal)
    for n, a, r in zip(("dq", "dk", "dv"), got, (rdq, rdk, rdv)):
        if np.linalg.norm(r) > 1e-6:
            e = rel_fro(host(a), r)
            report(f"stored-dS B={B} Lq={Lq} Lk={Lk} H={H} {n}", rel_fro=e)
            assert e <= GRAD_REL_FRO, (n, e)
        else:  # dS = 0 exactly (e.g. one query seeing one key): rounding error only
            e = float(np.abs(host(a) - r).max())
            report(f"stored-dS B={B} Lq={Lq} Lk={Lk} H={H} {n}", max_abs=e)
            assert e <= 1e-3, (n, e)


@pytest.mark.parametrize("L", [1, 64, 255, 300, 513])
def test_causal_ragged(L):
    stored_vs_recomputed(1, L, L, 2, 1 + L)


def test_noncausal_rectangular():
    stored_vs_recomputed(2, 700, 520, 3, 11, causal=False)


@pytest.mark.parametrize("q_offset,k_offset,Lq,Lk", [(180, 0, 520, 700), (0, 100, 400, 380),
                                                      (10000, 9800, 300, 600), (5000, 0, 260, 200),
                                                      (0, 30, 64, 640), (37, 0, 300, 300)])
def test_causal_offsets(q_offset, k_offset, Lq, Lk):
    stored_vs_recomputed(1, Lq, Lk, 2, 21 + Lq, q_offset=q_offset, k_offset=k_offset)


@pytest.mark.parametrize("seed", [31, 32])
def test_packed_segments(seed):
    stored_vs_recomputed(2, 1000, 1000, 2, seed, segs=True)


def test_segments_with_offsets():
    stored_vs_recomputed(1, 600, 900, 2, 41, segs=True, q_offset=300, k_offset=0)


def test_passes_of_eight_heads():
    # 16 pairs: one pass of all, two passes of 8; 12 pairs: passes of 8 and 4
    stored_vs_recomputed(1, 600, 600, 16, 51, heads=(None, 8))
    stored_vs_recomputed(2, 300, 300, 6, 52, heads=(8, 12))


def test_rope_fused_backward():
    need_gpu()
    B, L, H, seed = 1, 500, 2, 61
    note(f"stored dS, fused RoPE backward L={L}")
    q, k, v, do, _, _ = inputs(B, L, L, H, seed, False)
    qd, kd, vd, dod = dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), dev(do, "bf16")
    o, lse, q_rot, k_rot = lwm.lwm_blockattn_fwd_rope(qd, kd, vd, 1e6)
    ref = lwm.lwm_blockattn_bwd_rope(q_rot, k_rot, vd, o, lse, dod, 1e6,
                                     workspace=lwm.bwd_workspace(B, H, L, L, 128, "cuda", 0))
    ws = poisoned_workspace(B, H, L, L, None)
    got, n = stored_launches(lambda: lwm.lwm_blockattn_bwd_rope(q_rot, k_rot, vd, o, lse, dod, 1e6, workspace=ws))
    assert n == 1
    for name, a, r in zip(("dq", "dk", "dv"), got, ref):
        assert torch.equal(a, r), name


@pytest.mark.parametrize("segs", [False, True])
def test_ring_backward_stored_ds(segs):
    need_gpu()
    n, S, Lq, q_off, H, seed = 4, 160, 160, 480, 2, 71
    note(f"stored dS, backward ring n={n} shard={S} segs={segs}")
    q = synth.normal(seed, "q", (1, Lq, H, 128))
    do = synth.normal(seed, "do", (1, Lq, H, 128))
    k = synth.normal(seed, "k", (1, n * S, H, 128))
    v = synth.normal(seed, "v", (1, n * S, H, 128))
    seg = synth.random_segment_ids(seed, 1, n * S, 90) if segs else None
    qd, dod = dev(q, "bf16"), dev(do, "bf16")
    kd = [dev(k[:, j * S:(j + 1) * S], "bf16") for j in range(n)]
    vd = [dev(v[:, j * S:(j + 1) * S], "bf16") for j in range(n)]
    sqd = None if seg is None else seg_dev(seg[:, q_off:q_off + Lq])
    skd = None if seg is None else [seg_dev(seg[:, j * S:(j + 1) * S]) for j in range(n)]
    order = [3, 2, 1, 0]
    o, _, lse = path.ring_forward(qd, kd, vd, order, S, q_off, seg_q=sqd, seg_k_shards=skd)
    ref = path.ring_backward(qd, kd, vd, o, lse, dod, order, S, q_off, seg_q=sqd, seg_k_shards=skd,
                             workspace=lwm.bwd_workspace(1, H, Lq, S, 128, "cuda", 0))
    ws = poisoned_workspace(1, H, Lq, S, None, causal=False)
    got, n = stored_launches(lambda: path.ring_backward(qd, kd, vd, o, lse, dod, order, S, q_off, seg_q=sqd,
                                                        seg_k_shards=skd, workspace=ws))
    assert n == 4  # every shard is visible to the block (it sits after them all)
    assert torch.equal(got[0], ref[0]), "dq"
    for j in range(n):
        assert torch.equal(got[1][j], ref[1][j]), ("dk", j)
        assert torch.equal(got[2][j], ref[2][j]), ("dv", j)


def test_small_workspace_takes_the_recomputing_path():
    """A workspace one byte short of a slot per pair (B*H < 8) runs the recomputing path, which
    needs nothing beyond the two rows: poisoning the rest changes nothing."""
    need_gpu()
    B, L, H, seed = 1, 300, 2, 81
    note("stored dS: short workspace")
    q, k, v, do, _, _ = inputs(B, L, L, H, seed, False)
    qd, kd, vd, dod = dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), dev(do, "bf16")
    o, lse = lwm.lwm_blockattn_fwd(qd, kd, vd)
    full = lwm.lwm_blockattn_bwd_workspace_size_ds(B, H, L, L, 128, H)
    ws = torch.full((full - 1,), 255, dtype=torch.uint8, device="cuda")
    got, n = stored_launches(lambda: lwm.lwm_blockattn_bwd(qd, kd, vd, o, lse, dod, workspace=ws))
    assert n == 0
    ref = lwm.lwm_blockattn_bwd(qd, kd, vd, o, lse, dod, workspace=lwm.bwd_workspace(B, H, L, L, 128, "cuda", 0))
    torch.cuda.synchronize()
    for name, a, r in zip(("dq", "dk", "dv"), got, ref):
        assert torch.equal(a, r), name
