"""Helpers for the GPU parity tests: exact host<->device transfer of the seeded inputs."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

from ring_causal_attention_amd import synth


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def note(msg: str):
    """Name the case on stdout before any GPU work (flushed, so a fault still shows it)."""
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def report(case: str, **values):
    """Print the errors a parity check measured (shown with pytest -s), one line per check."""
    txt = " ".join(f"{k}={v:.3g}" if isinstance(v, float) else f"{k}={v}" for k, v in values.items())
    print(f"[parity] {case} {txt}", flush=True)


def dev(x: np.ndarray, dtype: str) -> torch.Tensor:
    """float32 host array -> device tensor; bf16 rounds to nearest even exactly like synth."""
    if dtype == "bf16":
        bits = synth.to_bf16_bits(x)
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def exact_host(x: np.ndarray, dtype: str) -> np.ndarray:
    """The float64 values the device sees for a float32 host array."""
    return (synth.round_to_bf16(x) if dtype == "bf16" else np.asarray(x, np.float32)).astype(np.float64)


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def seg_dev(seg: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.array(seg, dtype=np.int32, order="C")).cuda()  # a writable copy


def seg_pair_dev(sq, sk, seed):
    """Device segment ids for the two sides.  When both are the same ids, even seeds pass one
    tensor for both (the library's one-array path for packed self-attention), odd seeds two
    copies (its general path)."""
    if sq is None:
        return None, None
    if seed % 2 == 0 and sq.shape == sk.shape and np.array_equal(sq, sk):
        d = seg_dev(sq)
        return d, d
    return seg_dev(sq), seg_dev(sk)


def errors(got: np.ndarray, ref: np.ndarray):
    d = np.abs(got - ref)
    return float(d.max()) if d.size else 0.0, float(d.mean()) if d.size else 0.0


def rel_fro(got: np.ndarray, ref: np.ndarray) -> float:
    return float(np.linalg.norm((got - ref).ravel()) / max(np.linalg.norm(ref.ravel()), 1e-300))


# Tolerances on N(0,1) inputs (bf16 and fp32 forward; gradients by relative Frobenius norm).
BF16_MAX_ABS, BF16_MEAN_ABS = 2e-2, 2e-3
FP32_MAX_ABS = 1e-4
GRAD_REL_FRO = 1e-2
LSE_BF16, LSE_FP32 = 1e-2, 1e-5
