"""The matrix-core rate probe (lwm_probe_mfma_bf16) performs the products it is timed for.

Per wave, the sum of its lanes' sink values is the sum of all elements of its four final
accumulators.  The sum over all elements of a 32x16 by 16x32 product A B is
sum_k (sum_m A[m, k]) (sum_n B[k, n]); for v_mfma_f32_32x32x16_bf16 lane l supplies row (or
column) l % 32 of the operand and the 8 values of k = 8 (l // 32) .. + 7, so that sum follows
from per-half column sums of the lanes' fragments, with no assumption about the accumulator's
lane layout.  The check therefore pins the count of MFMAs per wave (iters rounds of four chains)
and the fragment rotation, which is what the timing depends on.
"""
import numpy as np
import pytest
import torch

from ring_causal_attention_amd import lwm

pytestmark = pytest.mark.gpu


def expected_wave_sums(src: np.ndarray, iters: int) -> np.ndarray:
    x = src.astype(np.float64).reshape(-1, 64, 16, 8)  # waves, lanes, fragments (8 A then 8 B), values
    a, b = x[:, :, :8, :], x[:, :, 8:, :]
    # initial accumulators: element i of chain c holds fragment (c + i) % 8, value i % 8
    init = np.zeros(x.shape[0])
    for c in range(4):
        for i in range(16):
            init += a[:, :, (c + i) % 8, i % 8].sum(axis=1)
    # per lane half h: sums over its 32 lanes of each fragment's 8 values -> [waves, frag, h, j]
    ah = np.stack([a[:, :32].sum(axis=1), a[:, 32:].sum(axis=1)], axis=2)
    bh = np.stack([b[:, :32].sum(axis=1), b[:, 32:].sum(axis=1)], axis=2)
    per_round = np.zeros(x.shape[0])
    for k in range(8):
        for c in range(4):
            per_round += (ah[:, (k + c) % 8] * bh[:, (3 * c + k) % 8]).sum(axis=(1, 2))
    return init + (iters // 8) * per_round


@pytest.mark.parametrize("blocks,iters", [(1, 8), (3, 64)])
def test_probe_products(blocks, iters):
    n = blocks * 256 * 128
    g = torch.Generator().manual_seed(1000 + blocks)
    # positive values: no cancellation in the sums, so a relative bound applies
    src = (0.5 + torch.rand(n, generator=g)).to(torch.bfloat16)
    sink = lwm.lwm_probe_mfma_bf16(src.cuda(), iters)
    torch.cuda.synchronize()
    got = sink.double().cpu().numpy().reshape(-1, 64).sum(axis=1)
    want = expected_wave_sums(src.float().numpy(), iters)
    np.testing.assert_allclose(got, want, rtol=1e-4)


def test_probe_zero_operands():
    sink = lwm.lwm_probe_mfma_bf16(torch.zeros(2 * 256 * 128, dtype=torch.bfloat16, device="cuda"), 16)
    torch.cuda.synchronize()
    assert torch.count_nonzero(sink).item() == 0
