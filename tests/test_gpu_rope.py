"""lwm_rope_apply against the oracle's RoPE (element by element)."""
import numpy as np
import pytest

import oracle
from ring_causal_attention_amd import lwm, synth
from tests.gpu_utils import dev, exact_host, host, need_gpu, note, seg_dev

pytestmark = pytest.mark.gpu


def _tol(dtype, ref):
    # bf16: rounding of the result (half an ulp, 2^-9 relative) plus float32 trigonometry
    return (np.abs(ref) * 2.0 ** -8 + 2e-6) if dtype == "bf16" else (np.abs(ref) * 1e-6 + 2e-6)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("layout", ["half", "interleaved"])
@pytest.mark.parametrize("mode", ["plain", "offset", "segments", "explicit"])
@pytest.mark.parametrize("inverse", [False, True])
def test_rope_parity(dtype, layout, mode, inverse):
    need_gpu()
    B, L, H, D = 2, 131, 3, 128
    theta = {"plain": 1.0e4, "offset": 5.0e7, "segments": 1.0e6, "explicit": 1.0e6}[mode]
    note(f"rope dtype={dtype} layout={layout} mode={mode} inverse={inverse}")
    x = synth.normal(7, "q", (B, L, H, D))
    xd = dev(x, dtype)
    kw, pos = {}, None
    if mode == "plain":
        pos = oracle.positions(B, L)
    elif mode == "offset":
        kw["pos_offset"] = 1_031_000
        pos = oracle.positions(B, L, 1_031_000)
    elif mode == "segments":
        seg = synth.random_segment_ids(3, B, L, 20)
        kw["seg"] = seg_dev(seg)
        kw["pos_offset"] = 5
        pos = oracle.positions(B, L, 5, seg)
    else:
        p = np.random.default_rng(5).integers(0, 1 << 20, size=(B, L)).astype(np.int32)
        kw["pos"] = seg_dev(p)
        pos = p.astype(np.int64)
    y = lwm.lwm_rope_apply(xd, theta=theta, layout=layout, inverse=inverse, **kw)
    ref = oracle.rope(exact_host(x, dtype), pos, theta, layout, inverse)
    got = host(y)
    assert np.all(np.abs(got - ref) <= _tol(dtype, ref)), float(np.max(np.abs(got - ref)))


def test_rope_in_place_and_strided():
    need_gpu()
    note("rope in place on a strided view")
    import torch
    B, L, H, D = 1, 64, 4, 128
    x = synth.normal(8, "k", (B, L, H, D))
    big = torch.zeros((B, L, H + 2, D), dtype=torch.bfloat16, device="cuda")
    view = big[:, :, 1:H + 1, :]
    view.copy_(dev(x, "bf16"))
    lwm.lwm_rope_apply(view, view, theta=1.0e6)
    ref = oracle.rope(exact_host(x, "bf16"), oracle.positions(B, L), 1.0e6)
    got = host(view)
    assert np.all(np.abs(got - ref) <= _tol("bf16", ref))
    assert float(big[:, :, 0].abs().sum()) == 0.0 and float(big[:, :, H + 1].abs().sum()) == 0.0


def test_rope_round_trip_at_one_million():
    need_gpu()
    note("rope forward then inverse at positions near 2^20, theta 5e7")
    B, L, H, D = 1, 96, 2, 128
    x = synth.normal(9, "q", (B, L, H, D))
    xd = dev(x, "fp32")
    y = lwm.lwm_rope_apply(xd, pos_offset=1_048_000, theta=5.0e7)
    z = lwm.lwm_rope_apply(y, pos_offset=1_048_000, theta=5.0e7, inverse=True)
    assert np.max(np.abs(host(z) - x.astype(np.float64))) < 1e-5


@pytest.mark.parametrize("layout", ["half", "interleaved"])
def test_rope_short_segments(layout):
    """Segments of 1 to 4 tokens, so segment starts fall at every offset inside the groups of
    tokens a workgroup rotates together, and ids that jump (non-consecutive values)."""
    need_gpu()
    B, L, H, D = 2, 203, 2, 128
    note(f"rope short segments layout={layout}")
    x = synth.normal(11, "q", (B, L, H, D))
    seg = synth.random_segment_ids(12, B, L, 4) * 3 + 1
    y = lwm.lwm_rope_apply(dev(x, "bf16"), theta=1.0e6, layout=layout, seg=seg_dev(seg), pos_offset=2)
    ref = oracle.rope(exact_host(x, "bf16"), oracle.positions(B, L, 2, seg), 1.0e6, layout)
    got = host(y)
    assert np.all(np.abs(got - ref) <= _tol("bf16", ref)), float(np.max(np.abs(got - ref)))
