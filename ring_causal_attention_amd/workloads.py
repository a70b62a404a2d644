"""Seeded host inputs for the five workloads, and their device copies (no attention arithmetic).

The ring workload generates only the K/V shards its query shard can see (0 .. ring_index): the
shards after it are in the causal future and the ring loop never reads them.
"""
from __future__ import annotations

import numpy as np
import torch

from . import synth
from .configs import Workload


def host_inputs(w: Workload, threads: int = 8) -> dict:
    """float32 N(0,1) arrays per tensor (shards as lists), segment ids, and RoPE offsets."""
    shape_q = (w.B, w.Lq, w.H, w.D)
    out: dict = {"workload": w}
    if w.ring_shards:
        vis = list(range(w.ring_index + 1))
        reqs = [(w.seed, "q", shape_q, None), (w.seed, "do", shape_q, None)]
        reqs += [(w.seed, t, (w.B, w.Lq, w.H, w.D), j) for t in ("k", "v") for j in vis]
        arrs = synth.normal_many(reqs, threads)
        out["q"], out["do"] = arrs[0], arrs[1]  # dO: upstream gradient of the backward ring
        n = len(vis)
        out["k_shards"] = dict(zip(vis, arrs[2:2 + n]))
        out["v_shards"] = dict(zip(vis, arrs[2 + n:2 + 2 * n]))
        out["seg"] = None
        return out
    names = ["q", "k", "v"] + (["do"] if w.backward else [])
    arrs = synth.normal_many([(w.seed, t, shape_q if t in ("q", "do") else (w.B, w.Lk, w.H, w.D), None)
                              for t in names], threads)
    out.update(dict(zip(names, arrs)))
    out["seg"] = synth.segment_ids_from_lengths(w.segment_lengths(), w.B) if w.packed else None
    return out


def to_device(x: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(synth.to_bf16_bits(x).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device)


def device_inputs(h: dict, device="cuda") -> dict:
    w: Workload = h["workload"]
    d: dict = {"workload": w}
    for name in ("q", "k", "v", "do"):
        if name in h:
            d[name] = to_device(h[name], w.dtype, device)
    for name in ("k_shards", "v_shards"):
        if name in h:
            d[name] = {j: to_device(x, w.dtype, device) for j, x in h[name].items()}
    d["seg"] = None if h["seg"] is None else torch.from_numpy(np.array(h["seg"], dtype=np.int32)).to(device)
    return d
