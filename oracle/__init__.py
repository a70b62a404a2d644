"""CPU oracle (float64 numpy) for blockwise causal ring attention with RoPE and packing.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py``; never by the product path.  See ``attention.py``
for the definitions, their sources and the readings taken where the sources are silent.
"""
from .attention import (  # noqa: F401
    NEG_INF,
    attention_bwd,
    attention_fwd,
    inv_freq,
    merge,
    positions,
    ring_step_bwd,
    rope,
    segment_positions,
    training_step,
    visible,
)
from .ffn import blockwise_ffn, silu, swiglu_ffn  # noqa: F401
