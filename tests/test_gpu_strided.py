"""Strided operands: Q, K, V (and their gradients, O, the ring state) as views into fused buffers,
the layout a fused QKV projection produces, against the oracle."""
import numpy as np
import pytest
import torch

import oracle
from ring_causal_attention_amd import lwm, path, synth
from tests.gpu_utils import (BF16_MAX_ABS, BF16_MEAN_ABS, GRAD_REL_FRO, LSE_BF16, dev, errors, exact_host, host,
                             need_gpu, note, rel_fro)

pytestmark = pytest.mark.gpu


def fused(seed, B, L, H):
    """float32 host arrays q, k, v and one device bf16 buffer [B, L, 3, H, 128] holding them."""
    q, k, v = (synth.normal(seed, t, (B, L, H, 128)) for t in ("q", "k", "v"))
    buf = dev(np.stack([q, k, v], axis=2), "bf16")
    return q, k, v, buf


@pytest.mark.parametrize("B,L,H", [(2, 300, 3), (1, 513, 5)])
def test_forward_and_backward_on_fused_views(B, L, H):
    need_gpu()
    note(f"strided fused-QKV B={B} L={L} H={H}")
    q, k, v, buf = fused(3000 + L, B, L, H)
    qd, kd, vd = buf[:, :, 0], buf[:, :, 1], buf[:, :, 2]
    assert not qd.is_contiguous() and qd.stride(1) == 3 * H * 128
    out = torch.full((B, L, 2, H, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    o = out[:, :, 1]                                   # a strided output view
    _, lse = lwm.lwm_blockattn_fwd(qd, kd, vd, o=o)
    do = synth.normal(3000 + L, "do", (B, L, H, 128))
    grads = torch.full((B, L, 3, H, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    dq, dk, dv = grads[:, :, 0], grads[:, :, 1], grads[:, :, 2]
    lwm.lwm_blockattn_bwd(qd, kd, vd, o, lse, dev(do, "bf16"), dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    qe, ke, ve = (exact_host(x, "bf16") for x in (q, k, v))
    ro, rl = oracle.attention_fwd(qe, ke, ve, None, None, 0, 0, True)
    mx, mean = errors(host(o), ro)
    assert mx <= BF16_MAX_ABS and mean <= BF16_MEAN_ABS, (mx, mean)
    assert np.max(np.abs(host(lse) - rl)) <= LSE_BF16
    assert bool(torch.isnan(out[:, :, 0].float()).all())  # the neighbouring slot is untouched
    rdq, rdk, rdv = oracle.attention_bwd(qe, ke, ve, exact_host(do, "bf16"), None, None, 0, 0, True)
    for name, g, r in (("dq", dq, rdq), ("dk", dk, rdk), ("dv", dv, rdv)):
        e = rel_fro(host(g), r)
        assert e <= GRAD_REL_FRO, (name, e)


def test_ring_on_strided_shards_and_state():
    need_gpu()
    note("strided ring shards and float32 state")
    B, S, H, n, r = 1, 160, 2, 3, 2
    q, k, v, buf = fused(3100, B, n * S, H)
    qd = buf[:, r * S:(r + 1) * S, 0]
    kd = [buf[:, j * S:(j + 1) * S, 1] for j in range(n)]
    vd = [buf[:, j * S:(j + 1) * S, 2] for j in range(n)]
    state = torch.zeros((B, S, H, 2, 128), dtype=torch.float32, device="cuda")
    o_acc = state[:, :, :, 0]                          # strided float32 state (head stride 256)
    lse_acc = torch.full((B, H, S), float("-inf"), dtype=torch.float32, device="cuda")
    o, _, lse = path.ring_forward(qd, kd, vd, [2, 1, 0], S, r * S, o_acc=o_acc, lse_acc=lse_acc)
    torch.cuda.synchronize()
    assert not bool(state[:, :, :, 1].any())
    qe, ke, ve = (exact_host(x, "bf16") for x in (q, k, v))
    ro, rl = oracle.attention_fwd(qe[:, r * S:(r + 1) * S], ke, ve, None, None, r * S, 0, True)
    mx, mean = errors(host(o), ro)
    assert mx <= BF16_MAX_ABS and mean <= BF16_MEAN_ABS, (mx, mean)
    assert np.max(np.abs(host(lse) - rl)) <= LSE_BF16
