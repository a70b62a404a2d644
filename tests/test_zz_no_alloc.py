"""lwm_blockattn_bwd_noalloc (the backward with the library's static per-GPU workspace) against
lwm_blockattn_bwd with a caller-owned workspace: two calls in a row, the second smaller, each
bit-identical to the allocating entry point's gradients on the same inputs."""
import pytest
import torch

from ring_causal_attention_amd import lwm
from tests.gpu_utils import dev, need_gpu, note, seg_dev
from ring_causal_attention_amd import synth

pytestmark = pytest.mark.gpu


def case(seed, B, L, H, seg=None, q_offset=0):
    q, k, v, do = (dev(synth.normal(seed, t, (B, L, H, 128)), "bf16") for t in ("q", "k", "v", "do"))
    sd = None if seg is None else seg_dev(seg)
    o, lse = lwm.lwm_blockattn_fwd(q, k, v, seg_q=sd, seg_k=sd, q_offset=q_offset)
    ref = lwm.lwm_blockattn_bwd(q, k, v, o, lse, do, seg_q=sd, seg_k=sd, q_offset=q_offset)
    got = tuple(torch.full_like(x, float("nan")) for x in ref)
    lwm.lwm_blockattn_bwd_noalloc(q, k, v, o, lse, do, *got, seg_q=sd, seg_k=sd, q_offset=q_offset)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), got, ref):
        assert torch.equal(a, b), name
    return got


def test_noalloc_backward_matches_allocating_entry_point():
    need_gpu()
    note("noalloc backward: B=2 L=700 H=3 packed, then B=1 L=130 H=2")
    seg = synth.random_segment_ids(77, 2, 700, 300)
    case(8100, 2, 700, 3, seg=seg)
    case(8101, 1, 130, 2, q_offset=5)


def test_noalloc_backward_rejects_oversized_calls():
    need_gpu()
    q = torch.empty((1, 1 << 16, 33, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((1, 33, 1 << 16), dtype=torch.float32, device="cuda")
    with pytest.raises(lwm.LwmError, match="static workspace"):
        lwm.lwm_blockattn_bwd_noalloc(q, q, q, q, lse, q, q, q, q)
