"""Planted mistakes in the oracle (on the CPU) must each be caught by at least one pin.

Every mutant is a fresh copy of ``oracle/attention.py`` with one plausible bug written into
its source text (a dropped term, a wrong sign or index, a transposed operand).  Each must
fail at least one pin, which shows the pins constrain every part of the oracle.
"""
import os
import types

import pytest

from tests import oracle_pins

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = open(os.path.join(ROOT, "oracle", "attention.py"), encoding="utf-8").read()

# (name, exact text in the oracle, planted replacement)
MUTANTS = [
    ("inv_freq_missing_two", "-2.0 * i / dim", "-1.0 * i / dim"),
    ("rope_sign", "ra = a * c - b * s", "ra = a * c + b * s"),
    ("rope_inverse_ignored", "        s = -s\n", "        s = s\n"),
    ("rope_pairs_swapped", 'a, b = x[..., : D // 2], x[..., D // 2:]', 'b, a = x[..., : D // 2], x[..., D // 2:]'),
    ("strict_causal", "gk[None, :] <= gq[:, None]", "gk[None, :] < gq[:, None]"),
    ("offsets_swapped", "gq = np.asarray(rows, dtype=np.int64) + int(q_offset)",
     "gq = np.asarray(rows, dtype=np.int64) + int(k_offset)"),
    ("no_segment_mask", "vis &= np.asarray(seg_q_row)[rows][:, None] == np.asarray(seg_k_row)[None, :]", "pass"),
    ("scale_default_dropped", "scale = 1.0 / math.sqrt(D) if scale is None else float(scale)\n    rows",
     "scale = 1.0 if scale is None else float(scale)\n    rows"),
    ("max_not_subtracted_from_lse", "m + np.log(np.where(has, l, 1.0))", "np.log(np.where(has, l, 1.0))"),
    ("lse_log2", "m + np.log(np.where(has, l, 1.0))", "m + np.log2(np.where(has, l, 1.0))"),
    ("bwd_rowsum_term_dropped", "ds = p * (dp - d_i[:, None])", "ds = p * dp"),
    ("bwd_dv_uses_dq_side", "dvh[:lim] += p.T @ dob", "dvh[:lim] += p.T @ qb"),
    ("bwd_dk_transposed_operand", "dkh[:lim] += scale * (ds.T @ qb)", "dkh[:lim] += scale * (ds.T @ dob)"),
    ("bwd_dq_missing_scale", "dq[b, rr, h, :] = scale * (ds @ kh[:lim])", "dq[b, rr, h, :] = ds @ kh[:lim]"),
    ("merge_weights_swapped", "return ca * np.asarray(o_a, dtype=np.float64) + cb * np.asarray(o_b",
     "return cb * np.asarray(o_a, dtype=np.float64) + ca * np.asarray(o_b"),
    ("segment_positions_not_restarting", "                start = t\n", "                start = 0\n"),
    ("ring_bwd_lse_not_subtracted", "np.exp(s - np.where(has, lb, 0.0)[:, None])", "np.exp(s)"),
    ("ring_bwd_rowsum_from_zero_o", "ob = np.asarray(o[b, rr, h, :], dtype=np.float64)", "ob = np.zeros_like(dob)"),
    ("ring_bwd_mask_ignored", "p = np.where(vis & has[:, None],", "p = np.where(has[:, None],"),
    ("training_inverse_rope_forgotten", "dq = rope(dqr, pos_q, theta, layout, inverse=True)",
     "dq = rope(dqr, pos_q, theta, layout)"),
]


FFN_SRC = open(os.path.join(ROOT, "oracle", "ffn.py"), encoding="utf-8").read()

# the same for the feed-forward oracle (checked against its own pins)
FFN_MUTANTS = [
    ("ffn_gate_dropped", "h = silu(x @ np.asarray(w_gate, dtype=np.float64).T) * (x @", "h = 1.0 * (x @"),
    ("ffn_gate_and_up_swapped", "h = silu(x @ np.asarray(w_gate, dtype=np.float64).T) * (x @ np.asarray(w_up,",
     "h = silu(x @ np.asarray(w_up, dtype=np.float64).T) * (x @ np.asarray(w_gate,"),
    ("silu_is_sigmoid", "    return z * sig", "    return sig"),
    ("silu_negative_branch_wrong", "np.where(z >= 0, 1.0 / (1.0 + e), e / (1.0 + e))", "np.where(z >= 0, 1.0 / (1.0 + e), 1.0 / (1.0 + e))"),
    ("ffn_down_not_transposed", "y = h @ np.asarray(w_down, dtype=np.float64).T", "y = h @ np.asarray(w_down, dtype=np.float64).T[::-1]"),
    ("blockwise_last_chunk_dropped", "for r0 in range(0, M, max(1, int(chunk))):", "for r0 in range(0, M - 1, max(1, int(chunk))):"),
]


def mutant(old, new, src=SRC):
    assert src.count(old) >= 1, f"mutation anchor vanished: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new, 1), "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(name, old, new):
    mod = mutant(old, new)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(mod)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin caught the planted mistake {name}"


@pytest.mark.parametrize("name,old,new", FFN_MUTANTS, ids=[m[0] for m in FFN_MUTANTS])
def test_planted_ffn_mistake_is_caught(name, old, new):
    mod = mutant(old, new, FFN_SRC)
    caught = []
    for pin in oracle_pins.FFN_PINS:
        try:
            pin(mod)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin caught the planted mistake {name}"
