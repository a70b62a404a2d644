"""The hot path composed from the C ABI calls (orchestration only; every step runs in HIP).

* ``ring_forward``   - one device's share of RingAttention simulated on one GPU: the query block
  stays put while the KV shards are visited in ring order, each folded into the running
  (O, lse) state by ``lwm_ring_step`` ("开源巨兽LWM：如何用RingAttention撬动百万Token多模态世界",
  section 3.1: devices form a ring, KV blocks rotate, compute overlaps transfer).
* ``attention_forward`` - RoPE on Q and K, then the blockwise forward.
* ``training_step`` - RoPE, forward (saving lse), backward, and inverse RoPE of dQ', dK' so the
  gradients are w.r.t. the pre-RoPE Q and K.
* ``training_step_fused`` - the same step with RoPE inside the attention calls: the forward
  rotates Q as it loads it (K by one pass) and the backward rotates dQ', dK' back before storing.
"""
from __future__ import annotations

import torch

from . import lwm


def ring_forward(q_rot, k_shards, v_shards, shard_order, shard_len, q_offset, causal=True, scale=0.0,
                 seg_q=None, seg_k_shards=None, o_acc=None, lse_acc=None, o_final=None):
    """Fold KV shards into the query block's state in ``shard_order``.

    q_rot: [B, Lq, H, D] bf16 (rotated); k_shards / v_shards: sequences of [B, shard_len, H, D]
    (rotated K); shard j holds global keys [j*shard_len, (j+1)*shard_len).  Shards wholly in
    the causal future of the block are skipped.  Returns (o_final bf16, o_acc, lse_acc).
    """
    B, Lq, H, D = q_rot.shape
    if o_acc is None:
        o_acc = torch.zeros((B, Lq, H, D), dtype=torch.float32, device=q_rot.device)
    if lse_acc is None:
        lse_acc = torch.full((B, H, Lq), float("-inf"), dtype=torch.float32, device=q_rot.device)
    if o_final is None:
        o_final = torch.empty_like(q_rot)
    last_q = q_offset + Lq - 1
    visible = [j for j in shard_order if not (causal and j * shard_len > last_q)]
    for n, j in enumerate(visible):
        lwm.lwm_ring_step(q_rot, k_shards[j], v_shards[j], o_acc, lse_acc,
                          seg_q=seg_q, seg_k=None if seg_k_shards is None else seg_k_shards[j],
                          q_offset=q_offset, k_offset=j * shard_len, causal=causal, scale=scale,
                          o_final=o_final if n == len(visible) - 1 else None)
    if not visible:
        o_final.zero_()
    return o_final, o_acc, lse_acc


def ring_backward(q_rot, k_shards, v_shards, o, lse, dout, shard_order, shard_len, q_offset, causal=True,
                  scale=0.0, seg_q=None, seg_k_shards=None, dq_acc=None, dk_acc=None, dv_acc=None, workspace=None,
                  ds_heads=None):
    """Backward ring for one query block: visit the KV shards in ``shard_order`` and add each
    shard's share of the gradients into ``dq_acc`` (float32 [B, Lq, H, D]) and into the shard's
    own ``dk_acc[j]``, ``dv_acc[j]`` (float32 [B, shard_len, H, D]; on a ring these travel with
    the shard).  o and lse are the forward's results over all shards (``ring_forward``).  Shards
    wholly in the causal future of the block are skipped: they add zero.  Accumulators that are
    not given start at zero.  Without a ``workspace`` one is allocated with room for the stored
    dS of ``ds_heads`` pairs per pass (``lwm.bwd_workspace``).  Returns (dq_acc, dk_acc, dv_acc),
    the last two dicts by shard.
    """
    B, Lq, H, D = q_rot.shape
    dev = q_rot.device
    if dq_acc is None:
        dq_acc = torch.zeros((B, Lq, H, D), dtype=torch.float32, device=dev)
    dk_acc = {} if dk_acc is None else dk_acc
    dv_acc = {} if dv_acc is None else dv_acc
    if workspace is None:  # dense slots (causal=False): the steps differ in k_offset
        workspace = lwm.bwd_workspace(B, H, Lq, shard_len, D, dev, ds_heads, causal=False)
    last_q = q_offset + Lq - 1
    first = True  # the first visited shard writes the block's delta and rescaled lse; the rest reuse them
    for j in shard_order:
        if causal and j * shard_len > last_q:
            continue
        kj = k_shards[j]
        if j not in dk_acc:
            dk_acc[j] = torch.zeros(kj.shape, dtype=torch.float32, device=dev)
        if j not in dv_acc:
            dv_acc[j] = torch.zeros(kj.shape, dtype=torch.float32, device=dev)
        lwm.lwm_ring_step_bwd(q_rot, kj, v_shards[j], o, lse, dout, dq_acc, dk_acc[j], dv_acc[j], seg_q=seg_q,
                              seg_k=None if seg_k_shards is None else seg_k_shards[j], q_offset=q_offset,
                              k_offset=j * shard_len, causal=causal, scale=scale, workspace=workspace,
                              reuse_workspace=not first)
        first = False
    return dq_acc, dk_acc, dv_acc


def attention_forward(q, k, v, theta, seg=None, layout="half", causal=True, scale=0.0, q_offset=0, k_offset=0,
                      pos_q_offset=None, pos_k_offset=None):
    """RoPE(Q), RoPE(K), blockwise forward.  Positions restart per segment when ``seg`` is given."""
    pq = q_offset if pos_q_offset is None else pos_q_offset
    pk = k_offset if pos_k_offset is None else pos_k_offset
    qr = lwm.lwm_rope_apply(q, seg=seg, pos_offset=pq, theta=theta, layout=layout)
    kr = lwm.lwm_rope_apply(k, seg=seg, pos_offset=pk, theta=theta, layout=layout)
    o, lse = lwm.lwm_blockattn_fwd(qr, kr, v, seg_q=seg, seg_k=seg, q_offset=q_offset, k_offset=k_offset,
                                   causal=causal, scale=scale)
    return o, lse, qr, kr


class TrainStepBuffers:
    """Device buffers of one training step, allocated once and reused across steps.  The backward
    workspace has room for the stored dS of ``ds_heads`` pairs per pass (``lwm.bwd_workspace``)."""

    def __init__(self, q, k, ds_heads=None, causal=True):
        B, L, H, D = q.shape
        Lk = k.shape[1]
        self.qr = torch.empty_like(q)
        self.kr = torch.empty_like(k)
        self.o = torch.empty_like(q)
        self.lse = torch.empty((B, H, L), dtype=torch.float32, device=q.device)
        self.dq = torch.empty_like(q)
        self.dk = torch.empty_like(k)
        self.dv = torch.empty_like(k)
        self.workspace = lwm.bwd_workspace(B, H, L, Lk, D, q.device, ds_heads, causal=causal)


def training_step(q, k, v, dout, theta, seg=None, layout="half", causal=True, scale=0.0, buffers=None):
    """Forward + backward of RoPE + causal attention; returns (o, lse, dq, dk, dv).

    dq and dk are gradients w.r.t. the pre-RoPE q and k: the backward's dQ', dK' are rotated
    back in place by the inverse RoPE.
    """
    bufs = buffers if buffers is not None else TrainStepBuffers(q, k, causal=causal)
    lwm.lwm_rope_apply(q, bufs.qr, seg=seg, theta=theta, layout=layout)
    lwm.lwm_rope_apply(k, bufs.kr, seg=seg, theta=theta, layout=layout)
    lwm.lwm_blockattn_fwd(bufs.qr, bufs.kr, v, seg_q=seg, seg_k=seg, causal=causal, scale=scale, o=bufs.o, lse=bufs.lse)
    lwm.lwm_blockattn_bwd(bufs.qr, bufs.kr, v, bufs.o, bufs.lse, dout, seg_q=seg, seg_k=seg, causal=causal,
                          scale=scale, dq=bufs.dq, dk=bufs.dk, dv=bufs.dv, workspace=bufs.workspace)
    lwm.lwm_rope_apply(bufs.dq, bufs.dq, seg=seg, theta=theta, layout=layout, inverse=True)
    lwm.lwm_rope_apply(bufs.dk, bufs.dk, seg=seg, theta=theta, layout=layout, inverse=True)
    return bufs.o, bufs.lse, bufs.dq, bufs.dk, bufs.dv


def training_step_fused(q, k, v, dout, theta, seg=None, layout="half", causal=True, scale=0.0, buffers=None):
    """``training_step`` through the fused-RoPE entry points; returns (o, lse, dq, dk, dv).

    Positions restart per segment when ``seg`` is given.  Two calls (forward, backward) and five
    kernels instead of seven: no separate RoPE pass over Q and no inverse-RoPE passes over dQ and dK.
    """
    bufs = buffers if buffers is not None else TrainStepBuffers(q, k, causal=causal)
    restart = seg is not None
    lwm.lwm_blockattn_fwd_rope(q, k, v, theta, seg_q=seg, seg_k=seg, causal=causal, scale=scale, layout=layout,
                               restart=restart, o=bufs.o, lse=bufs.lse, q_rot=bufs.qr, k_rot=bufs.kr)
    lwm.lwm_blockattn_bwd_rope(bufs.qr, bufs.kr, v, bufs.o, bufs.lse, dout, theta, seg_q=seg, seg_k=seg, causal=causal,
                               scale=scale, layout=layout, restart=restart, dq=bufs.dq, dk=bufs.dk, dv=bufs.dv,
                               workspace=bufs.workspace)
    return bufs.o, bufs.lse, bufs.dq, bufs.dk, bufs.dv
