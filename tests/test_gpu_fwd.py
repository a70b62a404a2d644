"""lwm_blockattn_fwd against the oracle on small shapes spanning tiles and ragged tails."""
import numpy as np
import pytest
import torch

import oracle
from ring_causal_attention_amd import lwm, synth
from tests.gpu_utils import (BF16_MAX_ABS, BF16_MEAN_ABS, FP32_MAX_ABS, LSE_BF16, LSE_FP32, dev, errors,
                             exact_host, host, need_gpu, note, seg_dev, seg_pair_dev)

pytestmark = pytest.mark.gpu

LENGTHS = [1, 2, 3, 63, 64, 65, 127, 128, 129, 1000]


def run_case(dtype, B, Lq, Lk, H, seed, seg=None, q_offset=0, k_offset=0, causal=True, scale=0.0):
    note(f"fwd dtype={dtype} B={B} Lq={Lq} Lk={Lk} H={H} seg={seg is not None} q_off={q_offset} "
         f"k_off={k_offset} causal={causal} seed={seed}")
    q = synth.normal(seed, "q", (B, Lq, H, 128))
    k = synth.normal(seed, "k", (B, Lk, H, 128))
    v = synth.normal(seed, "v", (B, Lk, H, 128))
    sq = sk = None
    if seg is not None:
        sq, sk = seg
    sqd, skd = seg_pair_dev(sq, sk, seed)
    o, lse = lwm.lwm_blockattn_fwd(dev(q, dtype), dev(k, dtype), dev(v, dtype), sqd, skd, q_offset, k_offset, causal,
                                   scale)
    torch.cuda.synchronize()
    ro, rl = oracle.attention_fwd(exact_host(q, dtype), exact_host(k, dtype), exact_host(v, dtype), sq, sk,
                                  q_offset, k_offset, causal, None if scale == 0.0 else scale)
    go, gl = host(o), host(lse)
    mx, mean = errors(go, ro)
    if dtype == "bf16":
        assert mx <= BF16_MAX_ABS and mean <= BF16_MEAN_ABS, (mx, mean)
    else:
        assert mx <= FP32_MAX_ABS, mx
    fin = np.isfinite(rl)
    assert np.array_equal(fin, np.isfinite(gl)), "rows without visible keys must give lse = -inf"
    assert np.all(np.isneginf(gl[~fin]))
    if fin.any():
        assert np.max(np.abs(gl[fin] - rl[fin])) <= (LSE_BF16 if dtype == "bf16" else LSE_FP32)
    return go, gl


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("L", LENGTHS)
def test_causal_lengths(dtype, L):
    need_gpu()
    run_case(dtype, 1, L, L, 2, 100 + L)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("L", [65, 300, 1000])
def test_packed_segments(dtype, L):
    need_gpu()
    seg = synth.random_segment_ids(L, 2, L, 97)  # non-decreasing ids, runs of 1..97 tokens
    run_case(dtype, 2, L, L, 2, 200 + L, seg=(seg, seg))


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_single_token_segments_and_noncausal(dtype):
    need_gpu()
    L = 257
    seg = np.minimum(np.arange(L) // 3, 40)[None, :].astype(np.int32)  # length-3 runs, last one long
    run_case(dtype, 1, L, L, 2, 301, seg=(seg, seg))
    run_case(dtype, 1, L, L, 2, 302, seg=(seg, seg), causal=False)
    run_case(dtype, 1, 190, 77, 2, 303, causal=False)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("offsets", [(0, 0), (200, 0), (64, 64), (1000, 900), (0, 50), (333, 17)])
def test_offsets(dtype, offsets):
    need_gpu()
    qo, ko = offsets
    run_case(dtype, 1, 150, 270, 2, 400 + qo + ko, q_offset=qo, k_offset=ko)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("offsets", [(1 << 33, 1 << 33), ((1 << 33) + 300, 1 << 33), ((1 << 31) + 77, 0),
                                     (5, (1 << 31) + 3)])
def test_large_offsets(dtype, offsets):
    """Global positions far beyond 32 bits (diagonal at 2^33, queries 2^31 past the keys, keys 2^31
    past the queries)."""
    need_gpu()
    qo, ko = offsets
    run_case(dtype, 1, 170, 330, 2, 450 + (qo + ko) % 97, q_offset=qo, k_offset=ko)


def test_custom_scale_and_batch_heads():
    need_gpu()
    run_case("bf16", 3, 200, 200, 5, 501, scale=0.05)
    run_case("bf16", 2, 129, 129, 8, 502)  # B*H multiple of 8: XCD-grouped block order


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("seed", [511, 512])
def test_packed_heads_multiple_of_eight(dtype, seed):
    """Packed rows with B*H a multiple of 8: tile-major, XCD-grouped block order; the even seed
    passes one id tensor for both sides (the single-search path), the odd one two equal copies."""
    need_gpu()
    L = 611
    seg = synth.random_segment_ids(seed, 2, L, 140)
    run_case(dtype, 2, L, L, 4, seed, seg=(seg, seg))


def test_rows_with_no_visible_key():
    need_gpu()
    go, gl = run_case("bf16", 1, 100, 100, 2, 601, q_offset=0, k_offset=50)
    assert np.all(go[:, :50] == 0.0) and np.all(np.isneginf(gl[:, :, :50]))


def test_empty_inputs():
    need_gpu()
    note("fwd empty inputs")
    for Lq, Lk in [(0, 10), (10, 0)]:
        q = torch.zeros((1, Lq, 2, 128), dtype=torch.bfloat16, device="cuda")
        k = torch.zeros((1, Lk, 2, 128), dtype=torch.bfloat16, device="cuda")
        o, lse = lwm.lwm_blockattn_fwd(q, k, k)
        torch.cuda.synchronize()
        if Lq:
            assert float(o.float().abs().sum()) == 0.0 and bool(torch.isneginf(lse).all())


def test_segment_start_rows_return_v_exactly():
    need_gpu()
    note("segment-start rows equal their V row bit for bit")
    L, H = 512, 2
    lens = [1, 37, 100, 2, 180, 192]
    seg = synth.segment_ids_from_lengths(lens)
    q, k, v = (synth.normal(700, t, (1, L, H, 128)) for t in ("q", "k", "v"))
    o, _ = lwm.lwm_blockattn_fwd(dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), seg_dev(seg), seg_dev(seg))
    starts = np.cumsum([0] + lens[:-1])
    got = host(o)[0, starts]
    assert np.array_equal(got, exact_host(v, "bf16")[0, starts])


def test_deterministic():
    need_gpu()
    note("forward bitwise determinism")
    q, k, v = (dev(synth.normal(800, t, (1, 700, 4, 128)), "bf16") for t in ("q", "k", "v"))
    ref, refl = lwm.lwm_blockattn_fwd(q, k, v)
    for _ in range(5):
        o, l = lwm.lwm_blockattn_fwd(q, k, v)
        assert torch.equal(o, ref) and torch.equal(l, refl)


def test_nan_poisoned_outputs_are_overwritten():
    need_gpu()
    note("every output element written")
    q, k, v = (dev(synth.normal(900, t, (2, 333, 3, 128)), "bf16") for t in ("q", "k", "v"))
    o = torch.full_like(q, float("nan"))
    lse = torch.full((2, 3, 333), float("nan"), device="cuda")
    lwm.lwm_blockattn_fwd(q, k, v, o=o, lse=lse)
    torch.cuda.synchronize()
    assert not bool(torch.isnan(o).any()) and not bool(torch.isnan(lse).any())
