"""Seeded random configurations of the forward and backward against the oracle.

Each case draws batch, heads, both lengths (ragged, 1 to 700), both global offsets, causal or not,
and packed segment ids (sorted, a few to a dozen segments; the query and key sides drawn separately
when their lengths differ) from one fixed seed, so the set is the same on every run and a failure
names its case.  The fixed-shape tests cover the edges one at a time; these mix them."""
import numpy as np
import pytest

from tests.gpu_utils import need_gpu
from tests.test_gpu_bwd import bwd_case
from tests.test_gpu_fwd import run_case

pytestmark = pytest.mark.gpu

N_CASES = 48


def draw_cases(seed=20261203, n=N_CASES, hmax=3, lmax=700, seed0=5000):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        B = int(rng.integers(1, 3))
        H = int(rng.integers(1, hmax + 1))
        Lq = int(rng.integers(1, lmax + 1))
        Lk = Lq if rng.random() < 0.5 else int(rng.integers(1, lmax + 1))
        causal = bool(rng.random() < 0.75)
        q_offset = int(rng.integers(0, 601)) if rng.random() < 0.5 else 0
        k_offset = int(rng.integers(0, 601)) if rng.random() < 0.5 else 0
        seg = None
        if rng.random() < 0.5:
            nseg = int(rng.integers(1, 13))
            sq = np.sort(rng.integers(0, nseg, size=(B, Lq)), axis=1).astype(np.int32)
            sk = sq.copy() if Lk == Lq else np.sort(rng.integers(0, nseg, size=(B, Lk)), axis=1).astype(np.int32)
            seg = (sq, sk)
        cases.append(dict(B=B, H=H, Lq=Lq, Lk=Lk, causal=causal, q_offset=q_offset, k_offset=k_offset, seg=seg,
                          seed=seed0 + i))
    return cases


# a second draw with up to 4 heads (so B*H reaches 8, the XCD-grouped block orders) and up to
# 1100 rows (several 256-key workgroups of the dK/dV kernel)
CASES = draw_cases() + draw_cases(seed=20261206, n=24, hmax=4, lmax=1100, seed0=5500)


def case_id(c):
    return (f"B{c['B']}H{c['H']}q{c['Lq']}k{c['Lk']}{'c' if c['causal'] else 'n'}"
            f"o{c['q_offset']}-{c['k_offset']}{'s' if c['seg'] is not None else ''}")


@pytest.mark.parametrize("c", CASES, ids=[case_id(c) for c in CASES])
def test_forward_random_config(c):
    need_gpu()
    run_case("bf16", c["B"], c["Lq"], c["Lk"], c["H"], c["seed"], c["seg"], c["q_offset"], c["k_offset"],
             c["causal"])


@pytest.mark.parametrize("c", CASES[:16], ids=[case_id(c) for c in CASES[:16]])
def test_forward_fp32_random_config(c):
    need_gpu()
    run_case("fp32", c["B"], c["Lq"], c["Lk"], c["H"], c["seed"], c["seg"], c["q_offset"], c["k_offset"],
             c["causal"])


@pytest.mark.parametrize("c", CASES, ids=[case_id(c) for c in CASES])
def test_backward_random_config(c):
    need_gpu()
    bwd_case(c["B"], c["Lq"], c["Lk"], c["H"], c["seed"], c["seg"], c["q_offset"], c["k_offset"], c["causal"])


def draw_fused_cases(seed=20261204, n=16):
    """RoPE inside the calls: theta, pair layout, positions restarting per segment, position offsets."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        B, H, L = int(rng.integers(1, 3)), int(rng.integers(1, 4)), int(rng.integers(1, 501))
        seg = None
        if rng.random() < 0.5:
            nseg = int(rng.integers(1, 9))
            seg = np.sort(rng.integers(0, nseg, size=(B, L)), axis=1).astype(np.int32)
        cases.append(dict(B=B, H=H, L=L, seg=seg, restart=bool(seg is not None and rng.random() < 0.6),
                          theta=float(rng.choice([1e4, 1e6, 5e7])),
                          layout=str(rng.choice(["half", "interleaved"])),
                          causal=bool(rng.random() < 0.8),
                          q_offset=int(rng.integers(0, 300)) if rng.random() < 0.4 else 0,
                          k_offset=int(rng.integers(0, 300)) if rng.random() < 0.4 else 0,
                          qpo=int(rng.integers(0, 1 << 20)) if rng.random() < 0.5 else 0,
                          kpo=int(rng.integers(0, 1 << 20)) if rng.random() < 0.5 else 0,
                          seed=6000 + i))
    return cases


FUSED = draw_fused_cases()


@pytest.mark.parametrize("c", FUSED, ids=[f"B{c['B']}H{c['H']}L{c['L']}{c['layout'][0]}{'r' if c['restart'] else ''}"
                                          f"{'s' if c['seg'] is not None else ''}" for c in FUSED])
def test_fused_rope_random_config(c):
    need_gpu()
    from tests.test_gpu_rope_fused import fused_case
    fused_case(c["B"], c["L"], c["L"], c["H"], c["seed"], c["theta"], c["layout"], c["seg"], c["restart"],
               c["q_offset"], c["k_offset"], c["qpo"], c["kpo"], c["causal"])


def draw_ring_cases(seed=20261205, n=12):
    """Backward ring: shard count and size, query block length and global offset, packing."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        n_shards, shard = int(rng.integers(2, 9)), int(rng.integers(1, 301))
        Lq = int(rng.integers(1, 301))
        q_off = int(rng.integers(0, n_shards * shard + 1))
        cases.append(dict(n_shards=n_shards, shard=shard, Lq=Lq, q_off=q_off, segs=bool(rng.random() < 0.4),
                          seed=7000 + i))
    return cases


RING = draw_ring_cases()


@pytest.mark.parametrize("c", RING, ids=[f"n{c['n_shards']}x{c['shard']}q{c['Lq']}@{c['q_off']}{'s' if c['segs'] else ''}"
                                         for c in RING])
def test_ring_backward_random_config(c):
    need_gpu()
    from tests.test_gpu_ring_bwd import ring_bwd_case
    ring_bwd_case(c["seed"], c["n_shards"], c["shard"], c["Lq"], c["q_off"], segs=c["segs"])
