"""CPU oracle for the blockwise feed-forward network of the transformer around the attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` may import this module.  It shares no code with the HIP path and imports
nothing from it; it computes the plain definition in float64 numpy.

Sources (page title, then section):

* [LWM-README] "LWM：突破 100 万 Token 的开源大模型".  §配置参数: the feed-forward network, like
  self-attention, can be computed blockwise, in chunks of ``scan_mlp_chunk_size`` along the
  sequence (``scan_mlp`` switches it on); §脚本运行说明 gives ``scan_mlp_chunk_size=8192``;
  §运行 PyTorch 模型: the text models load as HF ``LlamaForCausalLM``.

The pages do not write the network out.  Readings taken here:

* the feed-forward block is the LLaMA one the PyTorch port loads: y = W_down (silu(W_gate x) *
  (W_up x)) with silu(z) = z / (1 + e^-z), no biases;
* weights use the ``nn.Linear`` layout, [out_features, in_features]: W_gate, W_up are
  [d_ff, d_model] and W_down is [d_model, d_ff];
* "blockwise" splits only the token axis: each chunk of rows goes through the whole block, so
  the result equals the unchunked one exactly (up to rounding).

Pinned by brute-force scalar loops, ``torch.nn.functional.silu`` with ``torch.matmul`` on CPU
float64, the identity silu(z) - silu(-z) = z, and chunk-size invariance.
"""
from __future__ import annotations

import numpy as np


def silu(z):
    """z * sigmoid(z) = z / (1 + exp(-z)), float64, evaluated without overflow."""
    z = np.asarray(z, dtype=np.float64)
    e = np.exp(-np.abs(z))
    sig = np.where(z >= 0, 1.0 / (1.0 + e), e / (1.0 + e))
    return z * sig


def swiglu_ffn(x, w_gate, w_up, w_down):
    """y = (silu(x W_gate^T) * (x W_up^T)) W_down^T for x [M, d_model]; returns (y, h)."""
    x = np.asarray(x, dtype=np.float64)
    h = silu(x @ np.asarray(w_gate, dtype=np.float64).T) * (x @ np.asarray(w_up, dtype=np.float64).T)
    y = h @ np.asarray(w_down, dtype=np.float64).T
    return y, h


def blockwise_ffn(x, w_gate, w_up, w_down, chunk: int):
    """The feed-forward block applied to consecutive chunks of ``chunk`` rows ([LWM-README]
    §配置参数, ``scan_mlp_chunk_size``); returns y [M, d_model]."""
    x = np.asarray(x, dtype=np.float64)
    M = x.shape[0]
    out = np.zeros((M, np.asarray(w_down).shape[0]), dtype=np.float64)
    for r0 in range(0, M, max(1, int(chunk))):
        out[r0:r0 + chunk] = swiglu_ffn(x[r0:r0 + chunk], w_gate, w_up, w_down)[0]
    return out
