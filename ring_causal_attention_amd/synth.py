"""Seeded synthetic inputs shared by the GPU path's tests/bench and by the oracle's tests.

This module draws random numbers and nothing else: it holds none of the attention,
RoPE or masking arithmetic, so that the HIP path and the CPU oracle can both consume
exactly the same input bits without sharing any code that computes a result.

Recipe (every tensor is its own counter-addressed numpy stream):

* ``rng = numpy.random.default_rng([seed, tensor_id])`` (or ``[seed, tensor_id, shard]``
  for the sharded K/V of the ring workload), tensor ids Q=0, K=1, V=2, dO=3, segments=4;
* values: ``rng.standard_normal(shape, dtype=float32)`` in ``[B, L, H, D]`` order, i.e.
  N(0, 1), the distribution the workloads name; for bf16 workloads the float32 draw is
  rounded to bfloat16 with round-to-nearest-even (``to_bf16_bits``) and both sides see
  the identical bf16 values;
* feed-forward inputs (tensor ids x=5, W_gate=6, W_up=7, W_down=8): x is N(0, 1) (the block
  sees RMS-normalised activations), weights are N(0, 1) draws times ``w_std`` = 0.02 (the usual
  LLaMA initialisation scale; the pages give none), every array rounded to bfloat16;
* segments (masked sequence packing, "LWM：突破 100 万 Token 的开源大模型" §概述 item (b), and
  the packing bullet of "[论文解读] World Model on Million-Length Video And Language With
  Blockwise RingAttention" §提出的方法): integer lengths drawn uniformly from an inclusive
  range, one at a time, until they cover the row; the last one is cut to what remains.
  Ids are 0, 1, 2, ... in order, so they are non-decreasing along the row.
"""
from __future__ import annotations

import numpy as np

TENSOR_IDS = {"q": 0, "k": 1, "v": 2, "do": 3, "seg": 4, "x": 5, "w_gate": 6, "w_up": 7, "w_down": 8}


def normal(seed: int, tensor: str, shape, shard: int | None = None) -> np.ndarray:
    """float32 N(0,1) draw for one tensor (or one shard of it)."""
    key = [int(seed), TENSOR_IDS[tensor]] if shard is None else [int(seed), TENSOR_IDS[tensor], int(shard)]
    rng = np.random.default_rng(key)
    return rng.standard_normal(tuple(shape), dtype=np.float32)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round-to-nearest-even); returns the uint16 bit patterns.

    Works on the 32-bit patterns: adding 0x7FFF plus the lowest kept bit and truncating is
    round-to-nearest-even for every finite value (no finite pattern overflows 32 bits).
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    out = np.empty(u.shape, dtype=np.uint16)
    flat_u, flat_o = u.reshape(-1), out.reshape(-1)
    step = 1 << 24
    for i in range(0, flat_u.size, step):
        c = flat_u[i:i + step]
        r = (c >> 16) & 1
        r += c
        r += 0x7FFF
        flat_o[i:i + step] = r >> 16
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 values that are exactly representable in bfloat16 (RNE of the input)."""
    return bf16_bits_to_f32(to_bf16_bits(x))


def ffn_inputs(seed: int, rows: int, d_model: int, d_ff: int, w_std: float = 0.02, threads: int = 8) -> dict:
    """float32 arrays holding bf16-representable values: x [rows, d_model], w_gate and w_up
    [d_ff, d_model], w_down [d_model, d_ff]."""
    reqs = [(seed, "x", (rows, d_model), None), (seed, "w_gate", (d_ff, d_model), None),
            (seed, "w_up", (d_ff, d_model), None), (seed, "w_down", (d_model, d_ff), None)]
    arrs = normal_many(reqs, threads)
    out = {"x": round_to_bf16(arrs[0])}
    for name, a in zip(("w_gate", "w_up", "w_down"), arrs[1:]):
        a *= np.float32(w_std)
        out[name] = round_to_bf16(a)
    return out


def segment_lengths(seed: int, total: int, lo: int, hi: int) -> list[int]:
    """Packed-row segment lengths: uniform integers in [lo, hi], last one truncated."""
    rng = np.random.default_rng([int(seed), TENSOR_IDS["seg"]])
    out: list[int] = []
    covered = 0
    while covered < total:
        n = int(rng.integers(lo, hi, endpoint=True))
        n = min(n, total - covered)
        out.append(n)
        covered += n
    return out


def segment_ids_from_lengths(lengths, batch: int = 1) -> np.ndarray:
    """int32 [batch, sum(lengths)] ids 0, 1, 2, ... repeated per segment (same for every row)."""
    ids = np.repeat(np.arange(len(lengths), dtype=np.int32), np.asarray(lengths, dtype=np.int64))
    return np.ascontiguousarray(np.broadcast_to(ids, (batch, ids.shape[0])))


def random_segment_ids(seed: int, batch: int, length: int, max_len: int) -> np.ndarray:
    """Small random packings for tests: per batch row, lengths uniform in [1, max_len]."""
    rng = np.random.default_rng([int(seed), TENSOR_IDS["seg"], 7])
    out = np.zeros((batch, length), dtype=np.int32)
    for b in range(batch):
        t = 0
        sid = 0
        while t < length:
            n = int(rng.integers(1, max_len, endpoint=True))
            out[b, t:t + n] = sid
            t += n
            sid += 1
    return out


def normal_many(requests, threads: int = 8) -> list[np.ndarray]:
    """Several ``normal`` draws in parallel threads; ``requests`` holds (seed, tensor, shape, shard)."""
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        return list(ex.map(lambda r: normal(*r), requests))
