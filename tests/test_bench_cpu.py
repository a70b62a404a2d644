"""bench.py's host logic on the CPU: the settled timing of the extra lines and the accounting."""
import time
import types

import pytest

import bench
from ring_causal_attention_amd import configs

pytestmark = pytest.mark.cpu


def _fakes():
    calls = {"sync": 0, "reset": 0}
    torch = types.SimpleNamespace(cuda=types.SimpleNamespace(synchronize=lambda: calls.__setitem__("sync", calls["sync"] + 1)))
    lwm = types.SimpleNamespace(lwm_profile_reset=lambda: calls.__setitem__("reset", calls["reset"] + 1),
                                lwm_profile_enable=lambda on: None, lwm_profile_read=lambda: {})
    return torch, lwm, calls


def test_time_settled_raises_short_steps():
    torch, lwm, _ = _fakes()
    n = {"steps": 0}

    def step():
        n["steps"] += 1
        time.sleep(0.01)

    ms, prof, k, w = bench.time_settled(step, 3, 1, lwm, torch, warm_ms=60.0, timed_ms=120.0)
    # about 10 ms per step: warm-up covers about 60 ms and the timed part about 120 ms
    assert 3 <= w <= 7 and 6 <= k <= 13, (w, k)
    assert n["steps"] == 1 + w + k
    assert 9.0 <= ms <= 40.0


def test_time_settled_keeps_long_steps():
    torch, lwm, _ = _fakes()
    ms, prof, k, w = bench.time_settled(lambda: time.sleep(0.03), 2, 1, lwm, torch, warm_ms=20.0, timed_ms=40.0)
    assert (k, w) == (2, 1)


def test_kernel_work_accounting():
    w = configs.WORKLOADS["train_step_L32768"]
    pairs, D = w.visible_pairs(), w.D
    assert bench.kernel_work(w, "bwd_dkdv")[0] == 8 * D * pairs
    assert bench.kernel_work(w, "bwd_dq")[0] == 2 * D * pairs
    assert bench.kernel_work(w, "attn_fwd_bf16")[0] == 4 * D * pairs
    # forward + backward credited flop: 4D + 10D per pair
    credited = bench.kernel_work(w, "attn_fwd_bf16")[0] + bench.kernel_work(w, "bwd_dkdv")[0] + \
        bench.kernel_work(w, "bwd_dq")[0]
    assert credited == w.total_flop()
    assert bench.kernel_work(w, "rope_bf16") == (0, 2 * w.tensor_bytes())
