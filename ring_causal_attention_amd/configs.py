"""Workloads and algorithmic accounting (host logic only; no attention arithmetic).

Five workloads, each a synthetic N(0,1) input of the shape the pages' setting implies:

* ``causal_fp32_L1024``  - one causal sequence, L=1024, 4 heads, D=128, fp32, theta=1e4,
  forward only, one segment (the small parity case);
* ``llama7b_fwd_L32768`` - a LLaMA-7B attention layer forward (the pages' models are
  LLaMA-2-7B based): B=1, L=32768, 32 heads, D=128, bf16, theta=1e6, causal;
* ``packed_L65536``      - masked sequence packing: one packed row of 65536 tokens, segment
  lengths uniform in [256, 8192], block-diagonal causal mask, positions restart per segment;
* ``ring_share_1M``      - one device's share of a 1M-token ring (sequence axis 64, tensor
  axis 4 -> 8 of 32 heads): query shard of 16384 tokens at shard index 40, K/V as 64
  shards of 16384 visited in ring order with global offsets, theta=5e7;
* ``train_step_L32768``  - the llama7b shape forward + backward with upstream dO.

Counting follows the method: only visible (query, key) pairs of each head are counted, a
forward pair costs 4*D flop (QK^T and PV, 2*D each) and a backward pair 10*D flop (five
products: S, dP, dV, dK, dQ).
"""
from __future__ import annotations

import dataclasses

from . import synth


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    B: int
    Lq: int
    Lk: int
    H: int
    D: int
    dtype: str            # "bf16" | "fp32"
    theta: float
    causal: bool = True
    backward: bool = False
    packed: bool = False  # segment lengths uniform in [seg_lo, seg_hi]
    seg_lo: int = 256
    seg_hi: int = 8192
    ring_shards: int = 0  # > 0: K/V are ring_shards shards of Lq tokens, the query shard is ring_index
    ring_index: int = 0

    # -------------------------------------------------------------- segments / offsets
    def segment_lengths(self) -> list[int]:
        if not self.packed:
            return [self.Lq]
        return synth.segment_lengths(self.seed, self.Lq, self.seg_lo, self.seg_hi)

    @property
    def q_offset(self) -> int:
        return self.ring_index * self.Lq if self.ring_shards else 0

    def ring_order(self) -> list[int]:
        """Shards in the order the query device receives them: its own first, then r-1, r-2, ..."""
        n, r = self.ring_shards, self.ring_index
        return [(r - s) % n for s in range(n)]

    # -------------------------------------------------------------- accounting
    def visible_pairs_per_head(self) -> int:
        if self.ring_shards:
            s = self.Lq
            return self.ring_index * s * s + s * (s + 1) // 2
        if not self.causal:
            return sum(n * n for n in self.segment_lengths()) if self.packed else self.Lq * self.Lk
        return sum(n * (n + 1) // 2 for n in self.segment_lengths())

    def visible_pairs(self) -> int:
        return self.B * self.H * self.visible_pairs_per_head()

    def fwd_flop(self) -> int:
        return 4 * self.D * self.visible_pairs()

    def bwd_flop(self) -> int:
        return 10 * self.D * self.visible_pairs() if self.backward else 0

    def total_flop(self) -> int:
        return self.fwd_flop() + self.bwd_flop()

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4

    def tensor_bytes(self, L: int | None = None) -> int:
        return self.B * (self.Lq if L is None else L) * self.H * self.D * self.elem_bytes

    def fwd_bytes(self) -> int:
        """Bytes the forward must move once: Q, the visible K and V, O and lse (fp32)."""
        if self.ring_shards:
            kv = 2 * (self.ring_index + 1) * self.tensor_bytes()
        else:
            kv = 2 * self.tensor_bytes(self.Lk)
        return self.tensor_bytes() * 2 + kv + 4 * self.B * self.H * self.Lq


WORKLOADS = {
    w.name: w for w in [
        Workload("causal_fp32_L1024", 1001, 1, 1024, 1024, 4, 128, "fp32", 1.0e4),
        Workload("llama7b_fwd_L32768", 1002, 1, 32768, 32768, 32, 128, "bf16", 1.0e6),
        Workload("packed_L65536", 1003, 1, 65536, 65536, 32, 128, "bf16", 1.0e6, packed=True),
        Workload("ring_share_1M", 1004, 1, 16384, 16384, 8, 128, "bf16", 5.0e7, ring_shards=64, ring_index=40),
        Workload("train_step_L32768", 1005, 1, 32768, 32768, 32, 128, "bf16", 1.0e6, backward=True),
    ]
}

@dataclasses.dataclass(frozen=True)
class FfnWorkload:
    """The blockwise feed-forward block after each attention layer: `rows` tokens through a
    LLaMA-7B SwiGLU block (d_model 4096, d_ff 11008), `chunk` rows at a time."""
    name: str
    seed: int
    rows: int
    d_model: int
    d_ff: int
    chunk: int

    def flop(self) -> int:
        """Three products of rows x d_model x d_ff, 2 flop per multiply-add."""
        return 6 * self.rows * self.d_model * self.d_ff


FFN_WORKLOADS = {
    w.name: w for w in [
        FfnWorkload("ffn_llama7b_L32768", 1006, 32768, 4096, 11008, 8192),
    ]
}

# MI355X (gfx950) published peaks used for roofline fractions.
PEAK_BF16_TFLOPS = 2516.6     # 256 CU x 4096 flop/clk x 2.4 GHz (AMD's "2.5 PFLOP/s" dense bf16)
PEAK_FP32_MFMA_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
