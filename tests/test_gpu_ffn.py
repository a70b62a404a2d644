"""lwm_blockwise_ffn against the oracle's blockwise feed-forward block.

Tolerance, from the arithmetic: the HIP path accumulates in float32 and rounds h = silu(g) * u
to bf16 once (relative error below 2^-9, about 1.1e-3 rms) and y once more.  On the seeded
inputs each y element carries a rounding error of about 1.1e-3 * rms(y) from h plus its own
2^-9 relative rounding, so the relative Frobenius error of y stays near 1.6e-3; the test allows
1e-2, and per element 1e-2 * rms(y) + 2^-7 * |y|.
"""
import numpy as np
import pytest
import torch

import oracle
from ring_causal_attention_amd import configs, lwm, synth
from tests.gpu_utils import dev, host, need_gpu, note, rel_fro

pytestmark = pytest.mark.gpu

REL_FRO = 1e-2


def _dev_all(h):
    return {k: dev(v, "bf16") for k, v in h.items()}


def _check(got, ref):
    assert np.all(np.isfinite(got))
    assert rel_fro(got, ref) <= REL_FRO, rel_fro(got, ref)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    bad = np.abs(got - ref) > 1e-2 * rms + 2.0 ** -7 * np.abs(ref)
    assert not bad.any(), (np.argwhere(bad)[:5], float(np.abs(got - ref).max()), rms)


@pytest.mark.parametrize("rows,d_model,d_ff,chunk", [
    (1, 32, 32, 8192),        # one row, one K slab, one partial tile
    (130, 96, 160, 64),       # ragged row and column tiles, three chunks with a short last one
    (300, 256, 384, 128),     # several K slabs and column tiles
    (257, 4096, 352, 100),    # the model width along K, ragged chunk boundaries
    (1000, 512, 11008, 333),  # the model's d_ff (86 column tiles), chunks not tile-aligned
])
def test_ffn_parity(rows, d_model, d_ff, chunk):
    need_gpu()
    note(f"ffn rows={rows} d_model={d_model} d_ff={d_ff} chunk={chunk}")
    h = synth.ffn_inputs(31, rows, d_model, d_ff)
    d = _dev_all(h)
    y = lwm.lwm_blockwise_ffn(d["x"], d["w_gate"], d["w_up"], d["w_down"], chunk=chunk)
    torch.cuda.synchronize()
    ref = oracle.blockwise_ffn(h["x"], h["w_gate"], h["w_up"], h["w_down"], chunk)
    _check(host(y), ref)


def test_ffn_chunking_is_row_local():
    """Each row's result is the same whatever chunk it falls in (same products, same order)."""
    need_gpu()
    note("ffn chunk invariance rows=777 d_model=256 d_ff=512")
    h = synth.ffn_inputs(32, 777, 256, 512)
    d = _dev_all(h)
    ys = [lwm.lwm_blockwise_ffn(d["x"], d["w_gate"], d["w_up"], d["w_down"], chunk=c) for c in (777, 256, 100, 1)]
    torch.cuda.synchronize()
    for y in ys[1:]:
        assert torch.equal(y, ys[0])


def test_ffn_strided_views_and_fused_weights():
    """x and y as column slices of wider buffers; W_gate and W_up as halves of one fused weight."""
    need_gpu()
    rows, d_model, d_ff = 200, 128, 256
    note(f"ffn strided rows={rows} d_model={d_model} d_ff={d_ff}")
    h = synth.ffn_inputs(33, rows, d_model, d_ff)
    xw = torch.zeros((rows, d_model + 64), dtype=torch.bfloat16, device="cuda")
    xw[:, 32:32 + d_model] = dev(h["x"], "bf16")
    fused = torch.cat([dev(h["w_gate"], "bf16"), dev(h["w_up"], "bf16")], dim=0)
    wd = torch.zeros((d_model, d_ff + 16), dtype=torch.bfloat16, device="cuda")
    wd[:, :d_ff] = dev(h["w_down"], "bf16")
    yw = torch.full((rows, d_model + 40), 7.0, dtype=torch.bfloat16, device="cuda")
    lwm.lwm_blockwise_ffn(xw[:, 32:32 + d_model], fused[:d_ff], fused[d_ff:], wd[:, :d_ff], chunk=64,
                          y=yw[:, 8:8 + d_model])
    torch.cuda.synchronize()
    ref = oracle.blockwise_ffn(h["x"], h["w_gate"], h["w_up"], h["w_down"], 64)
    _check(host(yw[:, 8:8 + d_model]), ref)
    assert torch.all(yw[:, :8] == 7.0) and torch.all(yw[:, 8 + d_model:] == 7.0)


def test_ffn_degenerate_inputs():
    """Zero input or zero W_up gives exactly zero; rows = 0 writes nothing."""
    need_gpu()
    note("ffn degenerate inputs")
    h = synth.ffn_inputs(34, 96, 64, 96)
    d = _dev_all(h)
    y = lwm.lwm_blockwise_ffn(torch.zeros_like(d["x"]), d["w_gate"], d["w_up"], d["w_down"], chunk=64)
    assert torch.all(y == 0)
    y = lwm.lwm_blockwise_ffn(d["x"], d["w_gate"], torch.zeros_like(d["w_up"]), d["w_down"], chunk=64)
    assert torch.all(y == 0)
    e = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    assert lwm.lwm_blockwise_ffn(e, d["w_gate"], d["w_up"], d["w_down"]).shape == (0, 64)
    # saturated gates: silu(g) -> g for large g, -> 0 for very negative g (no NaN from exp overflow)
    x = torch.ones((32, 64), dtype=torch.bfloat16, device="cuda")
    wg = torch.full((96, 64), 4.0, dtype=torch.bfloat16, device="cuda")
    wg[48:] = -4.0
    wu = torch.full((96, 64), 1.0 / 64, dtype=torch.bfloat16, device="cuda")
    wd = torch.full((64, 96), 1.0 / 64, dtype=torch.bfloat16, device="cuda")
    y = host(lwm.lwm_blockwise_ffn(x, wg, wu, wd, chunk=8))
    ref = oracle.blockwise_ffn(host(x), host(wg), host(wu), host(wd), 8)
    _check(y, ref)


@pytest.mark.slow
def test_ffn_full_size_sampled_rows():
    """The benchmarked shape (32768 tokens, d_model 4096, d_ff 11008, chunks of 8192), in the
    same launch configuration, with sampled rows (chunk edges included) against the oracle."""
    need_gpu()
    w = configs.FFN_WORKLOADS["ffn_llama7b_L32768"]
    note(f"ffn full size {w}")
    h = synth.ffn_inputs(w.seed, w.rows, w.d_model, w.d_ff)
    d = _dev_all(h)
    y = lwm.lwm_blockwise_ffn(d["x"], d["w_gate"], d["w_up"], d["w_down"], chunk=w.chunk)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    rows = sorted(set([0, 127, 128, w.chunk - 1, w.chunk, 2 * w.chunk + 1, w.rows - 1]
                      + rng.integers(0, w.rows, 41).tolist()))
    ref, _ = oracle.swiglu_ffn(h["x"][rows], h["w_gate"], h["w_up"], h["w_down"])
    _check(host(y[rows]), ref)
