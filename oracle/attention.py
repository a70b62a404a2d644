"""CPU oracle for blockwise causal (ring) attention with RoPE and a packing mask.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  It shares no code with the
HIP path and imports nothing from it; it computes the plain definition in float64 numpy,
materialising every visible score, so that a reader can check it against the pages by eye.

Sources (page title, then section):

* [LWM-README] "LWM：突破 100 万 Token 的开源大模型" (Chinese translation of the LWM
  README).  §概述: RingAttention training of an autoregressive model, masked sequence
  packing to mix sequence lengths.  §配置参数: self-attention computed in query and key
  chunks (``scan_query_chunk_size`` / ``scan_key_chunk_size``); ``mesh_dim`` with a
  sequence-parallel axis for RingAttention.  §脚本运行说明: ``theta`` is a per-model
  setting (an example uses theta = 50000000, max_sequence_length = 32768).
* [LWM-review] "[论文解读] World Model on Million-Length Video And Language With Blockwise
  RingAttention".  §提出的方法: RoPE extended by scaling theta with context length; masked
  sequence packing.
* [LWM-blog] "开源巨兽LWM：如何用RingAttention撬动百万Token多模态世界".  §3.1: the sequence is
  cut into blocks, devices form a ring, a device computes on one block while the next is
  in transit.
* [LWM-medium] "Inside Large World Model: UC Berkeley Multimodal Model that can Understand
  1 Hour Long Videos".  "Stage I": RingAttention's block-wise computation; "Core
  Architecture": an autoregressive transformer.

None of the pages writes the attention formula.  What is computed here is the textbook
definition of causal softmax attention, which blockwise and ring evaluation reach exactly
(up to rounding order).  The readings taken where the pages are silent:

* scores are ``q . k / sqrt(D)`` (no bias, no soft-cap);
* "autoregressive" = key j is visible to query i iff ``global_k(j) <= global_q(i)``
  (the diagonal is visible), global index = shard offset + local index;
* packing mask: additionally ``seg_q(i) == seg_k(j)``;
* a row with no visible key has O = 0 and lse = -inf;
* lse is the natural-log logsumexp of the scaled visible scores;
* RoPE: ``inv_freq_i = theta ** (-2 i / D)``, angle = position * inv_freq_i, pairs
  (i, i + D/2) ("half", the HF ``LlamaForCausalLM`` convention that [LWM-README]
  §运行 PyTorch 模型 says the text models load as) or (2i, 2i+1) ("interleaved");
  under packing the position restarts at each segment start;
* gradients dQ, dK are taken w.r.t. the pre-RoPE Q and K (RoPE is part of the op).

Every function here is pinned by tests that do not re-run this code: brute-force scalar
loops, closed forms, a library routine (``torch.nn.functional.scaled_dot_product_attention``
and ``torch.autograd`` on CPU float64), central finite differences, and exact invariants.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

NEG_INF = -np.inf


# ----------------------------------------------------------------------------------------
# RoPE  ([LWM-review] §提出的方法: theta scaled with context length; values of theta per
# model are a setting, [LWM-README] §脚本运行说明)
# ----------------------------------------------------------------------------------------
def inv_freq(theta: float, dim: int) -> np.ndarray:
    """inv_freq_i = theta^(-2i/D), i = 0 .. D/2-1, float64."""
    i = np.arange(dim // 2, dtype=np.float64)
    return np.power(np.float64(theta), -2.0 * i / dim)


def segment_positions(seg: np.ndarray) -> np.ndarray:
    """Position of each token inside its packed segment: t - (index of the segment's first token).

    A segment is a maximal run of equal ids along the row ([LWM-README] §概述, masked
    sequence packing).  Returns int64 with the shape of ``seg`` ([B, L] or [L]).
    """
    seg = np.asarray(seg)
    flat = seg.reshape(-1, seg.shape[-1])
    out = np.empty(flat.shape, dtype=np.int64)
    for b in range(flat.shape[0]):
        start = 0
        for t in range(flat.shape[1]):
            if t > 0 and flat[b, t] != flat[b, t - 1]:
                start = t
            out[b, t] = t - start
    return out.reshape(seg.shape)


def rope(x: np.ndarray, pos: np.ndarray, theta: float, layout: str = "half",
         inverse: bool = False) -> np.ndarray:
    """Rotate every (pair of) feature(s) of x [B, L, H, D] by angle pos * inv_freq.

    ``pos`` is [B, L] or [L] (any integer or float dtype); ``inverse`` rotates by -angle.
    """
    x = np.asarray(x, dtype=np.float64)
    B, L, H, D = x.shape
    pos = np.broadcast_to(np.asarray(pos, dtype=np.float64), (B, L))
    ang = pos[:, :, None] * inv_freq(theta, D)[None, None, :]        # [B, L, D/2]
    c = np.cos(ang)[:, :, None, :]
    s = np.sin(ang)[:, :, None, :]
    if inverse:
        s = -s
    if layout == "half":
        a, b = x[..., : D // 2], x[..., D // 2:]
    elif layout == "interleaved":
        a, b = x[..., 0::2], x[..., 1::2]
    else:
        raise ValueError(f"unknown RoPE layout {layout!r}")
    ra = a * c - b * s
    rb = a * s + b * c
    out = np.empty_like(x)
    if layout == "half":
        out[..., : D // 2], out[..., D // 2:] = ra, rb
    else:
        out[..., 0::2], out[..., 1::2] = ra, rb
    return out


# ----------------------------------------------------------------------------------------
# Visibility: causal ([LWM-medium] "Core Architecture": autoregressive) and packing mask
# ([LWM-README] §概述 (b)) in global (shard-offset) coordinates ([LWM-blog] §3.1)
# ----------------------------------------------------------------------------------------
def visible(rows: np.ndarray, lk: int, q_offset: int, k_offset: int, causal: bool,
            seg_q_row: np.ndarray | None, seg_k_row: np.ndarray | None) -> np.ndarray:
    """bool [len(rows), lk]: key j visible to query rows[r]."""
    gq = np.asarray(rows, dtype=np.int64) + int(q_offset)
    gk = np.arange(lk, dtype=np.int64) + int(k_offset)
    vis = np.ones((len(rows), lk), dtype=bool)
    if causal:
        vis &= gk[None, :] <= gq[:, None]
    if seg_q_row is not None:
        vis &= np.asarray(seg_q_row)[rows][:, None] == np.asarray(seg_k_row)[None, :]
    return vis


def _pool_map(fn, tasks, threads):
    if threads <= 1 or len(tasks) <= 1:
        return [fn(t) for t in tasks]
    with ThreadPoolExecutor(max_workers=threads) as ex:
        return list(ex.map(fn, tasks))


def _threads(threads):
    return max(1, int(threads if threads is not None else (os.cpu_count() or 1)))


def _softmax_block(qb, kh, vis, scale):
    """Scores, row max and normalised probabilities for one block of query rows."""
    s = (qb @ kh.T) * scale
    s = np.where(vis, s, NEG_INF)
    m = s.max(axis=1)
    has = np.isfinite(m)
    e = np.where(vis, np.exp(s - np.where(has, m, 0.0)[:, None]), 0.0)
    l = e.sum(axis=1)
    p = e / np.where(has, l, 1.0)[:, None]
    lse = np.where(has, m + np.log(np.where(has, l, 1.0)), NEG_INF)
    return p, lse


def _key_limit(rows, lk, q_offset, k_offset, causal):
    """Number of leading keys that can be visible to any of ``rows`` (causal trimming only)."""
    if not causal or len(rows) == 0:
        return lk
    last = int(np.max(rows)) + int(q_offset) - int(k_offset)
    return int(min(lk, max(0, last + 1)))


def attention_fwd(q, k, v, seg_q=None, seg_k=None, q_offset: int = 0, k_offset: int = 0,
                  causal: bool = True, scale: float | None = None, rows=None,
                  row_block: int = 512, threads: int | None = None):
    """softmax(Q K^T * scale + mask) V and its natural-log logsumexp, float64.

    q [B, Lq, H, D], k/v [B, Lk, H, D] (already rotated), seg_q [B, Lq], seg_k [B, Lk] or None.
    ``rows`` selects query rows (default: all).  Returns O [B, R, H, D], lse [B, H, R].
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    B, Lq, H, D = q.shape
    Lk = k.shape[1]
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    rows = np.arange(Lq) if rows is None else np.asarray(rows, dtype=np.int64)
    R = len(rows)
    o = np.zeros((B, R, H, D), dtype=np.float64)
    lse = np.full((B, H, R), NEG_INF, dtype=np.float64)

    def one(task):
        b, h = task
        kh = np.ascontiguousarray(k[b, :, h, :], dtype=np.float64)
        vh = np.ascontiguousarray(v[b, :, h, :], dtype=np.float64)
        for r0 in range(0, R, row_block):
            rr = rows[r0:r0 + row_block]
            lim = _key_limit(rr, Lk, q_offset, k_offset, causal)
            if lim == 0:
                continue
            qb = np.asarray(q[b, rr, h, :], dtype=np.float64)
            vis = visible(rr, lim, q_offset, k_offset, causal,
                          None if seg_q is None else seg_q[b], None if seg_k is None else seg_k[b][:lim])
            p, lb = _softmax_block(qb, kh[:lim], vis, scale)
            o[b, r0:r0 + len(rr), h, :] = p @ vh[:lim]
            lse[b, h, r0:r0 + len(rr)] = lb

    _pool_map(one, [(b, h) for b in range(B) for h in range(H)], _threads(threads))
    return o, lse


def attention_bwd(q, k, v, dout, seg_q=None, seg_k=None, q_offset: int = 0, k_offset: int = 0,
                  causal: bool = True, scale: float | None = None, row_block: int = 512,
                  threads: int | None = None, heads=None):
    """Gradients of sum(dout * O) w.r.t. q, k, v (the rotated operands), float64.

    With P the normalised probabilities: dV = P^T dO; dP = dO V^T; D_i = sum_d dO_id O_id;
    dS = P o (dP - D); dQ = scale dS K; dK = scale dS^T Q.  ``heads`` restricts the work to
    a subset of heads (others are left zero).  Returns dq, dk, dv with the input shapes.
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    dout = np.asarray(dout)
    B, Lq, H, D = q.shape
    Lk = k.shape[1]
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    dq = np.zeros((B, Lq, H, D), dtype=np.float64)
    dk = np.zeros((B, Lk, H, D), dtype=np.float64)
    dv = np.zeros((B, Lk, H, D), dtype=np.float64)
    heads = range(H) if heads is None else heads

    def one(task):
        b, h = task
        kh = np.ascontiguousarray(k[b, :, h, :], dtype=np.float64)
        vh = np.ascontiguousarray(v[b, :, h, :], dtype=np.float64)
        dkh = np.zeros((Lk, D))
        dvh = np.zeros((Lk, D))
        for r0 in range(0, Lq, row_block):
            rr = np.arange(r0, min(Lq, r0 + row_block))
            lim = _key_limit(rr, Lk, q_offset, k_offset, causal)
            if lim == 0:
                continue
            qb = np.asarray(q[b, rr, h, :], dtype=np.float64)
            dob = np.asarray(dout[b, rr, h, :], dtype=np.float64)
            vis = visible(rr, lim, q_offset, k_offset, causal,
                          None if seg_q is None else seg_q[b], None if seg_k is None else seg_k[b][:lim])
            p, _ = _softmax_block(qb, kh[:lim], vis, scale)
            ob = p @ vh[:lim]
            d_i = np.sum(dob * ob, axis=1)
            dvh[:lim] += p.T @ dob
            dp = dob @ vh[:lim].T
            ds = p * (dp - d_i[:, None])
            dq[b, rr, h, :] = scale * (ds @ kh[:lim])
            dkh[:lim] += scale * (ds.T @ qb)
        dk[b, :, h, :] = dkh
        dv[b, :, h, :] = dvh

    _pool_map(one, [(b, h) for b in range(B) for h in heads], _threads(threads))
    return dq, dk, dv


# ----------------------------------------------------------------------------------------
# Backward ring step ([LWM-blog] §3.1: each device keeps its query block while key/value
# blocks travel the ring; for the backward the gradients of a key/value block travel with it)
# ----------------------------------------------------------------------------------------
def ring_step_bwd(q, k, v, o, lse, dout, seg_q=None, seg_k=None, q_offset: int = 0, k_offset: int = 0,
                  causal: bool = True, scale: float | None = None, row_block: int = 512,
                  threads: int | None = None):
    """Contributions of one key/value shard to the gradients of sum(dout * O), float64.

    O [B, Lq, H, D] and lse [B, H, Lq] are the forward's final results over *all* shards, so
    P_ij = exp(S_ij * scale - lse_i) on this shard's visible keys is the exact probability and
    D_i = sum_d dO_id O_id is the full row term.  Returns (dq, dk, dv): dq [B, Lq, H, D] is this
    shard's share of dQ (summed over shards it gives dQ), dk / dv [B, Lk, H, D] are this query
    block's share of the shard's dK / dV (summed over query blocks they give dK / dV).
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    o = np.asarray(o)
    lse = np.asarray(lse)
    dout = np.asarray(dout)
    B, Lq, H, D = q.shape
    Lk = k.shape[1]
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    dq = np.zeros((B, Lq, H, D), dtype=np.float64)
    dk = np.zeros((B, Lk, H, D), dtype=np.float64)
    dv = np.zeros((B, Lk, H, D), dtype=np.float64)

    def one(task):
        b, h = task
        kh = np.ascontiguousarray(k[b, :, h, :], dtype=np.float64)
        vh = np.ascontiguousarray(v[b, :, h, :], dtype=np.float64)
        dkh = np.zeros((Lk, D))
        dvh = np.zeros((Lk, D))
        for r0 in range(0, Lq, row_block):
            rr = np.arange(r0, min(Lq, r0 + row_block))
            lim = _key_limit(rr, Lk, q_offset, k_offset, causal)
            if lim == 0:
                continue
            qb = np.asarray(q[b, rr, h, :], dtype=np.float64)
            dob = np.asarray(dout[b, rr, h, :], dtype=np.float64)
            ob = np.asarray(o[b, rr, h, :], dtype=np.float64)
            lb = np.asarray(lse[b, h, rr], dtype=np.float64)
            vis = visible(rr, lim, q_offset, k_offset, causal,
                          None if seg_q is None else seg_q[b], None if seg_k is None else seg_k[b][:lim])
            s = (qb @ kh[:lim].T) * scale
            has = np.isfinite(lb)
            p = np.where(vis & has[:, None], np.exp(s - np.where(has, lb, 0.0)[:, None]), 0.0)
            d_i = np.sum(dob * ob, axis=1)
            dvh[:lim] += p.T @ dob
            dp = dob @ vh[:lim].T
            ds = p * (dp - d_i[:, None])
            dq[b, rr, h, :] = scale * (ds @ kh[:lim])
            dkh[:lim] += scale * (ds.T @ qb)
        dk[b, :, h, :] = dkh
        dv[b, :, h, :] = dvh

    _pool_map(one, [(b, h) for b in range(B) for h in range(H)], _threads(threads))
    return dq, dk, dv


# ----------------------------------------------------------------------------------------
# Merge of two partial results over disjoint key sets (ring step; [LWM-blog] §3.1 rotates
# KV blocks around the ring, each visit contributes one partial softmax)
# ----------------------------------------------------------------------------------------
def merge(o_a, lse_a, o_b, lse_b):
    """Exact combination of (O, lse) pairs over disjoint key sets.

    O [B, R, H, D], lse [B, H, R].  M = max(lse_a, lse_b); lse = M + ln(e^(lse_a-M) + e^(lse_b-M));
    O = e^(lse_a-lse) O_a + e^(lse_b-lse) O_b; a side with lse = -inf weighs 0; both -inf give
    O = 0, lse = -inf.
    """
    lse_a = np.asarray(lse_a, dtype=np.float64)
    lse_b = np.asarray(lse_b, dtype=np.float64)
    m = np.maximum(lse_a, lse_b)
    has = np.isfinite(m)
    ms = np.where(has, m, 0.0)
    wa = np.where(np.isfinite(lse_a), np.exp(lse_a - ms), 0.0)
    wb = np.where(np.isfinite(lse_b), np.exp(lse_b - ms), 0.0)
    tot = wa + wb
    lse = np.where(has, ms + np.log(np.where(has, tot, 1.0)), NEG_INF)
    ca = np.where(has, wa / np.where(has, tot, 1.0), 0.0)   # [B, H, R]
    cb = np.where(has, wb / np.where(has, tot, 1.0), 0.0)
    ca = np.transpose(ca, (0, 2, 1))[..., None]             # -> [B, R, H, 1]
    cb = np.transpose(cb, (0, 2, 1))[..., None]
    return ca * np.asarray(o_a, dtype=np.float64) + cb * np.asarray(o_b, dtype=np.float64), lse


# ----------------------------------------------------------------------------------------
# Compositions used by the workloads
# ----------------------------------------------------------------------------------------
def positions(B: int, L: int, offset: int = 0, seg=None) -> np.ndarray:
    """[B, L] RoPE positions: offset + t, or offset + position inside the packed segment."""
    if seg is None:
        return np.broadcast_to(np.arange(L, dtype=np.int64) + int(offset), (B, L)).copy()
    return segment_positions(seg) + int(offset)


def training_step(q, k, v, dout, pos_q, pos_k, theta, layout="half", seg_q=None, seg_k=None,
                  q_offset=0, k_offset=0, causal=True, scale=None, threads=None):
    """RoPE -> attention forward -> backward -> gradients w.r.t. the pre-RoPE Q and K.

    Since R(pos) is orthogonal, d(loss)/dQ = R(pos)^-1 d(loss)/dQ'.  Returns o, lse, dq, dk, dv.
    """
    qr = rope(q, pos_q, theta, layout)
    kr = rope(k, pos_k, theta, layout)
    o, lse = attention_fwd(qr, kr, v, seg_q, seg_k, q_offset, k_offset, causal, scale, threads=threads)
    dqr, dkr, dv = attention_bwd(qr, kr, v, dout, seg_q, seg_k, q_offset, k_offset, causal, scale,
                                 threads=threads)
    dq = rope(dqr, pos_q, theta, layout, inverse=True)
    dk = rope(dkr, pos_k, theta, layout, inverse=True)
    return o, lse, dq, dk, dv
