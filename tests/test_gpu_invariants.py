"""Invariants on the GPU that need no oracle run: closed forms (constant V, Q = 0), a resumable
ring state, NaN-poisoned and canary-guarded outputs."""
import numpy as np
import pytest
import torch

from ring_causal_attention_amd import lwm, path, synth
from tests.gpu_utils import dev, exact_host, host, need_gpu, note, seg_dev

pytestmark = pytest.mark.gpu


def test_constant_v_returns_the_constant():
    need_gpu()
    note("constant V")
    B, L, H = 1, 333, 2
    q = dev(synth.normal(4000, "q", (B, L, H, 128)), "bf16")
    k = dev(synth.normal(4000, "k", (B, L, H, 128)), "bf16")
    c = np.linspace(-2.0, 2.0, 128, dtype=np.float32)
    v = dev(np.broadcast_to(c, (B, L, H, 128)).copy(), "bf16")
    o, _ = lwm.lwm_blockattn_fwd(q, k, v)
    torch.cuda.synchronize()
    ce = exact_host(c, "bf16")
    # the same bf16-rounded p weight O and l, so O is c up to float32 rounding and the bf16 store
    assert np.max(np.abs(host(o) - ce)) <= 2 ** -7


def test_zero_query_averages_the_visible_values():
    need_gpu()
    note("Q = 0: uniform weights over the visible keys")
    B, L, H = 1, 257, 2
    seg = synth.random_segment_ids(4100, B, L, 40)
    q = torch.zeros((B, L, H, 128), dtype=torch.bfloat16, device="cuda")
    k = dev(synth.normal(4100, "k", (B, L, H, 128)), "bf16")
    vh = synth.normal(4100, "v", (B, L, H, 128))
    o, lse = lwm.lwm_blockattn_fwd(q, k, dev(vh, "bf16"), seg_dev(seg), seg_dev(seg))
    torch.cuda.synchronize()
    ve = exact_host(vh, "bf16")
    ref = np.zeros_like(ve)
    cnt = np.zeros(L)
    for i in range(L):
        vis = [j for j in range(i + 1) if seg[0, j] == seg[0, i]]
        ref[0, i] = ve[0, vis].mean(axis=0)
        cnt[i] = len(vis)
    assert np.max(np.abs(host(o) - ref)) <= 2e-2
    assert np.max(np.abs(host(lse)[0] - np.log(cnt)[None, :])) <= 1e-5


def test_ring_state_resumes_bit_for_bit():
    need_gpu()
    note("ring: stop, keep the state, resume")
    n, S, H, r = 5, 96, 2, 4
    q = dev(synth.normal(4200, "q", (1, S, H, 128)), "bf16")
    k = [dev(synth.normal(4200, "k", (1, S, H, 128), shard=j), "bf16") for j in range(n)]
    v = [dev(synth.normal(4200, "v", (1, S, H, 128), shard=j), "bf16") for j in range(n)]
    order = [4, 3, 2, 1, 0]
    o_ref, acc_ref, lse_ref = path.ring_forward(q, k, v, order, S, r * S)
    acc = torch.zeros((1, S, H, 128), dtype=torch.float32, device="cuda")
    lse = torch.full((1, H, S), float("-inf"), dtype=torch.float32, device="cuda")
    path.ring_forward(q, k, v, order[:2], S, r * S, o_acc=acc, lse_acc=lse)
    saved = (acc.clone(), lse.clone())                # a complete checkpoint of the ring
    acc2, lse2 = saved[0].clone(), saved[1].clone()
    o2, _, _ = path.ring_forward(q, k, v, order[2:], S, r * S, o_acc=acc2, lse_acc=lse2)
    torch.cuda.synchronize()
    assert torch.equal(acc2, acc_ref) and torch.equal(lse2, lse_ref) and torch.equal(o2, o_ref)


def test_backward_overwrites_poisoned_gradients():
    need_gpu()
    note("backward: NaN-poisoned dq / dk / dv, rows and keys that see nothing")
    B, L, H = 1, 200, 2
    q, k, v, do = (dev(synth.normal(4300, t, (B, L, H, 128)), "bf16") for t in ("q", "k", "v", "do"))
    o, lse = lwm.lwm_blockattn_fwd(q, k, v, q_offset=0, k_offset=150)   # rows 0..149 see nothing
    dq, dk, dv = (torch.full_like(q, float("nan")) for _ in range(3))
    lwm.lwm_blockattn_bwd(q, k, v, o, lse, do, q_offset=0, k_offset=150, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    for t in (dq, dk, dv):
        assert not bool(torch.isnan(t).any())
    assert not bool(dq[:, :150].any())                 # no visible key: zero gradient
    assert not bool(dk[:, 50:].any()) and not bool(dv[:, 50:].any())  # keys from global 200 on: unseen


def test_outputs_stay_inside_their_views():
    need_gpu()
    note("canaries around o, lse and the backward outputs")
    B, L, H = 1, 130, 3
    q, k, v, do = (dev(synth.normal(4400, t, (B, L, H, 128)), "bf16") for t in ("q", "k", "v", "do"))
    guard = 7
    big = torch.full((B, L + 2 * guard, H, 128), 3.0, dtype=torch.bfloat16, device="cuda")
    o = big[:, guard:guard + L]
    lse_big = torch.full((B, H, L + 2 * guard), 5.0, dtype=torch.float32, device="cuda")
    lse = lse_big[:, :, guard:guard + L].contiguous()
    lwm.lwm_blockattn_fwd(q, k, v, o=o, lse=lse)
    grads = torch.full((3, B, L + 2 * guard, H, 128), 3.0, dtype=torch.bfloat16, device="cuda")
    dq, dk, dv = (grads[i, :, guard:guard + L] for i in range(3))
    lwm.lwm_blockattn_bwd(q, k, v, o, lse, do, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    for t in (big, grads[0], grads[1], grads[2]):
        assert bool((t[:, :guard] == 3.0).all()) and bool((t[:, guard + L:] == 3.0).all())
