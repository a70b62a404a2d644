"""Pins for the CPU oracle: checks that do not re-run the oracle's own code.

Each ``pin_*`` takes an oracle namespace (the real ``oracle`` package, or a mutant with a
planted mistake) and raises ``AssertionError`` when the oracle disagrees with something the
pages or mathematics fix independently: brute-force scalar loops, an independent complex
formulation of RoPE, closed forms, exact invariants, a library routine
(``torch.nn.functional.scaled_dot_product_attention`` and ``torch.autograd``, CPU float64)
or central finite differences.
"""
from __future__ import annotations

import cmath
import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(*key):
    return np.random.default_rng(list(key))


def _rand(rng, *shape):
    return rng.standard_normal(shape)


# ---------------------------------------------------------------- brute force (scalar loops)
def brute_fwd(q, k, v, seg_q, seg_k, q_offset, k_offset, causal, scale):
    """Pure-Python loops with math.fsum / math.exp: O and lse per row."""
    B, Lq, H, D = q.shape
    Lk = k.shape[1]
    o = np.zeros((B, Lq, H, D))
    lse = np.full((B, H, Lq), -math.inf)
    for b in range(B):
        for h in range(H):
            for i in range(Lq):
                keys = [j for j in range(Lk)
                        if (not causal or k_offset + j <= q_offset + i)
                        and (seg_q is None or int(seg_q[b][i]) == int(seg_k[b][j]))]
                if not keys:
                    continue
                s = [scale * math.fsum(float(q[b, i, h, d]) * float(k[b, j, h, d]) for d in range(D))
                     for j in keys]
                mx = max(s)
                e = [math.exp(x - mx) for x in s]
                tot = math.fsum(e)
                for d in range(D):
                    o[b, i, h, d] = math.fsum(e[t] * float(v[b, j, h, d]) for t, j in enumerate(keys)) / tot
                lse[b, h, i] = mx + math.log(tot)
    return o, lse


def brute_rope(x, pos, theta, layout, inverse):
    """RoPE as a complex multiplication z * exp(i * angle), one pair at a time."""
    B, L, H, D = x.shape
    out = np.zeros_like(x, dtype=np.float64)
    half = D // 2
    for b in range(B):
        for t in range(L):
            p = float(np.broadcast_to(pos, (B, L))[b, t])
            for h in range(H):
                for i in range(half):
                    ia, ib = (i, i + half) if layout == "half" else (2 * i, 2 * i + 1)
                    ang = p * (theta ** (-(2.0 * i) / D))
                    z = complex(x[b, t, h, ia], x[b, t, h, ib]) * cmath.exp(1j * (-ang if inverse else ang))
                    out[b, t, h, ia], out[b, t, h, ib] = z.real, z.imag
    return out


def _tiny_case(seed, B=2, Lq=7, Lk=9, H=2, D=6, segs=True, maxlen=4):
    rng = _rng(seed, 99)
    q, k, v = _rand(rng, B, Lq, H, D), _rand(rng, B, Lk, H, D), _rand(rng, B, Lk, H, D)
    seg_q = seg_k = None
    if segs:
        # keys and queries share one packed row in global coordinates
        n = max(Lq, Lk) + 8
        ids = np.zeros((B, n), dtype=np.int64)
        for b in range(B):
            t, sid = 0, 0
            while t < n:
                ln = int(rng.integers(1, maxlen + 1))
                ids[b, t:t + ln] = sid
                t += ln
                sid += 1
        return q, k, v, ids, ids
    return q, k, v, seg_q, seg_k


# ---------------------------------------------------------------- forward pins
def pin_forward_brute_force(orc):
    for seed, (qo, ko, causal, segs) in enumerate([(0, 0, True, False), (0, 0, True, True),
                                                   (5, 2, True, True), (3, 0, False, True),
                                                   (0, 4, True, False), (2, 2, False, False)]):
        q, k, v, sq, sk = _tiny_case(seed, segs=segs)
        if segs:
            # global coordinates: query i sits at qo + i, key j at ko + j in one packed row
            sq = sq[:, qo:qo + q.shape[1]]
            sk = sk[:, ko:ko + k.shape[1]]
        scale = 0.37 if seed % 2 else 1.0 / math.sqrt(q.shape[-1])
        o_ref, lse_ref = brute_fwd(q, k, v, sq, sk, qo, ko, causal, scale)
        o, lse = orc.attention_fwd(q, k, v, sq, sk, qo, ko, causal, scale, threads=1)
        assert np.allclose(o, o_ref, atol=1e-12, rtol=0), f"O mismatch case {seed}"
        fin = np.isfinite(lse_ref)
        assert np.array_equal(fin, np.isfinite(lse)), f"lse finiteness case {seed}"
        assert np.allclose(lse[fin], lse_ref[fin], atol=1e-12, rtol=0), f"lse mismatch case {seed}"
        assert np.all(o[np.transpose(~fin, (0, 2, 1))] == 0.0)
        # row subsets give the same rows
        rows = np.array([0, q.shape[1] - 1, 2])
        o2, l2 = orc.attention_fwd(q, k, v, sq, sk, qo, ko, causal, scale, rows=rows, threads=1)
        assert np.allclose(o2, o_ref[:, rows], atol=1e-12, rtol=0)


def pin_forward_sdpa(orc):
    """Library special case: torch SDPA (CPU float64) with an explicit boolean mask."""
    import torch
    import torch.nn.functional as F
    rng = _rng(11)
    B, L, H, D = 2, 150, 3, 32
    q, k, v = _rand(rng, B, L, H, D), _rand(rng, B, L, H, D), _rand(rng, B, L, H, D)
    seg = np.repeat(np.arange(6), [10, 33, 1, 50, 26, 30])[None, :].repeat(B, 0)
    for segs, causal in [(False, True), (True, True), (True, False)]:
        sq = sk = seg if segs else None
        mask = np.ones((B, L, L), dtype=bool)
        if causal:
            mask &= np.tril(np.ones((L, L), dtype=bool))[None]
        if segs:
            mask &= seg[:, :, None] == seg[:, None, :]
        t = lambda a: torch.from_numpy(np.ascontiguousarray(np.transpose(a, (0, 2, 1, 3))))
        ref = F.scaled_dot_product_attention(t(q), t(k), t(v), attn_mask=torch.from_numpy(mask)[:, None])
        ref = np.transpose(ref.numpy(), (0, 2, 1, 3))
        o, _ = orc.attention_fwd(q, k, v, sq, sk, 0, 0, causal, None, threads=2)
        assert np.allclose(o, ref, atol=1e-12, rtol=0), (segs, causal)


def pin_forward_closed_forms(orc):
    rng = _rng(12)
    B, L, H, D = 1, 40, 2, 16
    q, k, v = _rand(rng, B, L, H, D), _rand(rng, B, L, H, D), _rand(rng, B, L, H, D)
    seg = np.repeat(np.arange(4), [1, 12, 7, 20])[None, :]
    starts = [0, 1, 13, 20]
    scale = 1.0 / math.sqrt(D)
    o, lse = orc.attention_fwd(q, k, v, seg, seg, 0, 0, True, None, threads=1)
    # (i) a row whose only visible key is itself returns that V row, lse = its own score
    for s in starts:
        assert np.allclose(o[0, s], v[0, s], atol=1e-13, rtol=0)
        for h in range(H):
            assert abs(lse[0, h, s] - scale * float(np.dot(q[0, s, h], k[0, s, h]))) < 1e-12
    # (ii) Q = 0: O = mean of the visible V rows, lse = ln(#visible)
    o0, lse0 = orc.attention_fwd(np.zeros_like(q), k, v, seg, seg, 0, 0, True, None, threads=1)
    for i in range(L):
        st = max(s for s in starts if s <= i)
        assert np.allclose(o0[0, i], v[0, st:i + 1].mean(axis=0), atol=1e-13, rtol=0)
        assert np.allclose(lse0[0, :, i], math.log(i + 1 - st), atol=1e-13, rtol=0)
    # (iii) constant V returns that constant
    c = rng.standard_normal(D)
    vc = np.broadcast_to(c, v.shape).copy()
    oc, _ = orc.attention_fwd(q, k, vc, seg, seg, 0, 0, True, None, threads=1)
    assert np.allclose(oc, np.broadcast_to(c, oc.shape), atol=1e-13, rtol=0)


def pin_forward_invariants(orc):
    rng = _rng(13)
    B, L, H, D = 1, 64, 2, 16
    q, k, v = _rand(rng, B, L, H, D), _rand(rng, B, L, H, D), _rand(rng, B, L, H, D)
    o, lse = orc.attention_fwd(q, k, v, None, None, 0, 0, True, None, threads=1)
    # shifting every key by one vector c leaves O unchanged (a per-row constant in softmax)
    c = rng.standard_normal((1, 1, H, D))
    o2, _ = orc.attention_fwd(q, k + c, v, None, None, 0, 0, True, None, threads=1)
    assert np.allclose(o, o2, atol=1e-12, rtol=0)
    # causal prefix: rows < 40 of a length-64 run equal a length-40 run
    o3, lse3 = orc.attention_fwd(q[:, :40], k[:, :40], v[:, :40], None, None, 0, 0, True, None, threads=1)
    assert np.allclose(o[:, :40], o3, atol=1e-13, rtol=0)
    assert np.allclose(lse[:, :, :40], lse3, atol=1e-13, rtol=0)


def pin_packed_equals_unpacked(orc):
    """Each packed segment (positions restart) equals an unpacked causal run of it alone."""
    rng = _rng(14)
    lens = [5, 17, 1, 30, 11]
    L, H, D, theta = sum(lens), 2, 8, 1.0e4
    q, k, v = _rand(rng, 1, L, H, D), _rand(rng, 1, L, H, D), _rand(rng, 1, L, H, D)
    seg = np.repeat(np.arange(len(lens)), lens)[None, :]
    pos = orc.positions(1, L, 0, seg)
    qr, kr = orc.rope(q, pos, theta), orc.rope(k, pos, theta)
    o, lse = orc.attention_fwd(qr, kr, v, seg, seg, 0, 0, True, None, threads=1)
    t = 0
    for n in lens:
        sl = slice(t, t + n)
        pu = np.arange(n)
        ou, lu = orc.attention_fwd(orc.rope(q[:, sl], pu, theta), orc.rope(k[:, sl], pu, theta), v[:, sl],
                                   None, None, 0, 0, True, None, threads=1)
        assert np.allclose(o[:, sl], ou, atol=1e-12, rtol=0)
        assert np.allclose(lse[:, :, sl], lu, atol=1e-12, rtol=0)
        t += n


def pin_block_and_ring_invariance(orc):
    """Chunked keys merged in any order equal the full result; masked shards are no-ops."""
    rng = _rng(15)
    B, Lq, H, D = 1, 48, 2, 16
    n_shards, shard = 6, 32
    Lk = n_shards * shard
    q_off = 3 * shard + 5                     # the query block sits inside shard 3
    q = _rand(rng, B, Lq, H, D)
    k, v = _rand(rng, B, Lk, H, D), _rand(rng, B, Lk, H, D)
    full_o, full_l = orc.attention_fwd(q, k, v, None, None, q_off, 0, True, None, threads=1)
    parts = []
    for j in range(n_shards):
        sl = slice(j * shard, (j + 1) * shard)
        parts.append(orc.attention_fwd(q, k[:, sl], v[:, sl], None, None, q_off, j * shard, True, None,
                                       threads=1))
    orders = [list(range(n_shards)), list(range(n_shards))[::-1],
              [(3 - s) % n_shards for s in range(n_shards)], list(_rng(16).permutation(n_shards))]
    for order in orders:
        acc_o = np.zeros_like(full_o)
        acc_l = np.full_like(full_l, -np.inf)
        for j in order:
            acc_o, acc_l = orc.merge(acc_o, acc_l, *parts[j])
        assert np.allclose(acc_o, full_o, atol=1e-12, rtol=0), order
        assert np.allclose(acc_l, full_l, atol=1e-12, rtol=0), order
    # a fully masked shard (all keys in the future) is exactly a no-op
    o5, l5 = parts[5]
    assert np.all(np.isneginf(l5)) and np.all(o5 == 0)
    mo, ml = orc.merge(full_o, full_l, o5, l5)
    assert np.array_equal(mo, full_o) and np.array_equal(ml, full_l)
    # stop after three shards, save, resume: identical to an uninterrupted pass
    acc = (np.zeros_like(full_o), np.full_like(full_l, -np.inf))
    for j in (3, 2, 1):
        acc = orc.merge(*acc, *parts[j])
    saved = (acc[0].copy(), acc[1].copy())
    for j in (0, 5, 4):
        acc = orc.merge(*acc, *parts[j])
    res = saved
    for j in (0, 5, 4):
        res = orc.merge(*res, *parts[j])
    assert np.array_equal(acc[0], res[0]) and np.array_equal(acc[1], res[1])
    # chunk sizes named for the blockwise scan (128 / 512) on a longer row
    L2 = 1024
    q2, k2, v2 = _rand(rng, 1, L2, 1, 8), _rand(rng, 1, L2, 1, 8), _rand(rng, 1, L2, 1, 8)
    ref_o, ref_l = orc.attention_fwd(q2, k2, v2, None, None, 0, 0, True, None, threads=1)
    for chunk in (128, 512):
        acc = (np.zeros_like(ref_o), np.full_like(ref_l, -np.inf))
        for c0 in range(0, L2, chunk):
            acc = orc.merge(*acc, *orc.attention_fwd(q2, k2[:, c0:c0 + chunk], v2[:, c0:c0 + chunk],
                                                     None, None, 0, c0, True, None, threads=1))
        assert np.allclose(acc[0], ref_o, atol=1e-12, rtol=0)
        assert np.allclose(acc[1], ref_l, atol=1e-12, rtol=0)


# ---------------------------------------------------------------- RoPE pins
def pin_rope(orc):
    rng = _rng(17)
    # D = 2: inv_freq = 1, so a plain rotation by pos radians (closed form)
    x = _rand(rng, 1, 5, 1, 2)
    pos = np.array([0, 1, 2, 7, 1000])
    y = orc.rope(x, pos, 12345.0, "half")
    for t, p in enumerate(pos):
        c, s = math.cos(p), math.sin(p)
        a, b = x[0, t, 0]
        assert np.allclose(y[0, t, 0], [a * c - b * s, a * s + b * c], atol=1e-14, rtol=0)
    for layout in ("half", "interleaved"):
        B, L, H, D, theta = 2, 9, 3, 8, 500.0
        x = _rand(rng, B, L, H, D)
        pos = rng.integers(0, 2_000_000, size=(B, L))
        y = orc.rope(x, pos, theta, layout)
        assert np.allclose(y, brute_rope(x, pos, theta, layout, False), atol=1e-12, rtol=0)
        yi = orc.rope(x, pos, theta, layout, inverse=True)
        assert np.allclose(yi, brute_rope(x, pos, theta, layout, True), atol=1e-12, rtol=0)
        # position 0 is the identity; inverse(forward) is the identity
        assert np.allclose(orc.rope(x, np.zeros((B, L)), theta, layout), x, atol=0, rtol=0)
        assert np.allclose(orc.rope(y, pos, theta, layout, inverse=True), x, atol=1e-12, rtol=0)
        # the norm of every pair is preserved
        if layout == "half":
            na, nb = (x[..., :D // 2] ** 2 + x[..., D // 2:] ** 2), (y[..., :D // 2] ** 2 + y[..., D // 2:] ** 2)
        else:
            na, nb = (x[..., 0::2] ** 2 + x[..., 1::2] ** 2), (y[..., 0::2] ** 2 + y[..., 1::2] ** 2)
        assert np.allclose(na, nb, atol=1e-12, rtol=0)
    # relative-position identity <R_m q, R_n k> = <q, R_(n-m) k>
    D = 16
    qv, kv = _rand(rng, 1, 1, 1, D), _rand(rng, 1, 1, 1, D)
    for m, n in [(3, 10), (1000, 1007), (123456, 5)]:
        lhs = float(np.sum(orc.rope(qv, [m], 1e4) * orc.rope(kv, [n], 1e4)))
        rhs = float(np.sum(qv * orc.rope(kv, [n - m], 1e4)))
        assert abs(lhs - rhs) < 1e-9, (m, n)
    # inverse frequencies: theta^(-2i/D)
    f = orc.inv_freq(1.0e6, 128)
    assert f[0] == 1.0 and abs(f[32] - 1.0e-3) < 1e-18 and abs(f[-1] - 1.0e6 ** (-126 / 128)) < 1e-20


def pin_segment_positions(orc):
    seg = np.array([[0, 0, 0, 1, 2, 2, 5, 5, 5, 5], [3, 3, 3, 3, 3, 3, 3, 3, 3, 4]])
    expect = np.array([[0, 1, 2, 0, 0, 1, 0, 1, 2, 3], [0, 1, 2, 3, 4, 5, 6, 7, 8, 0]])
    assert np.array_equal(orc.segment_positions(seg), expect)
    assert np.array_equal(orc.positions(2, 10, 100, seg), expect + 100)
    assert np.array_equal(orc.positions(1, 4, 7), [[7, 8, 9, 10]])


# ---------------------------------------------------------------- backward pins
def pin_backward_finite_differences(orc):
    rng = _rng(18)
    B, L, H, D = 1, 5, 1, 4
    seg = np.array([[0, 0, 1, 1, 1]])
    q, k, v, do = (_rand(rng, B, L, H, D) for _ in range(4))
    dq, dk, dv = orc.attention_bwd(q, k, v, do, seg, seg, 0, 0, True, None, threads=1)

    def loss(qq, kk, vv):
        o, _ = brute_fwd(qq, kk, vv, seg, seg, 0, 0, True, 1.0 / math.sqrt(D))
        return float(np.sum(o * do))

    h = 1e-6
    for name, arr, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            a1, a2 = arr.copy(), arr.copy()
            a1[idx] += h
            a2[idx] -= h
            args1 = {"q": (a1, k, v), "k": (q, a1, v), "v": (q, k, a1)}[name]
            args2 = {"q": (a2, k, v), "k": (q, a2, v), "v": (q, k, a2)}[name]
            num[idx] = (loss(*args1) - loss(*args2)) / (2 * h)
        assert np.allclose(g, num, atol=2e-8, rtol=0), name


def pin_backward_autograd(orc):
    """Library check: torch.autograd through SDPA (CPU float64) with the same mask."""
    import torch
    import torch.nn.functional as F
    rng = _rng(19)
    B, L, H, D = 2, 70, 2, 16
    q, k, v, do = (_rand(rng, B, L, H, D) for _ in range(4))
    seg = np.repeat(np.arange(4), [20, 1, 30, 19])[None, :].repeat(B, 0)
    mask = np.tril(np.ones((L, L), dtype=bool))[None] & (seg[:, :, None] == seg[:, None, :])
    tt = [torch.tensor(np.transpose(a, (0, 2, 1, 3)), requires_grad=True) for a in (q, k, v)]
    out = F.scaled_dot_product_attention(*tt, attn_mask=torch.from_numpy(mask)[:, None])
    out.backward(torch.from_numpy(np.ascontiguousarray(np.transpose(do, (0, 2, 1, 3)))))
    ref = [np.transpose(t.grad.numpy(), (0, 2, 1, 3)) for t in tt]
    got = orc.attention_bwd(q, k, v, do, seg, seg, 0, 0, True, None, threads=2)
    for r, g, n in zip(ref, got, "qkv"):
        assert np.allclose(g, r, atol=1e-11, rtol=0), n


def pin_backward_identities(orc):
    rng = _rng(20)
    B, L, H, D = 1, 96, 2, 8
    q, k, v, do = (_rand(rng, B, L, H, D) for _ in range(4))
    q_off = 7
    o, lse = orc.attention_fwd(q, k, v, None, None, q_off, 0, True, None, threads=1)
    dq, dk, dv = orc.attention_bwd(q, k, v, do, None, None, q_off, 0, True, None, threads=1)
    # every row sees at least key 0 here: sum_j dV_j = sum_i dO_i
    assert np.allclose(dv.sum(axis=1), do.sum(axis=1), atol=1e-11, rtol=0)
    # rows of dS sum to zero, so sum_j dK_j = 0
    assert np.allclose(dk.sum(axis=1), 0.0, atol=1e-11, rtol=0)
    # O is linear in V: <dV, V> = <dO, O> per head
    for h in range(H):
        assert abs(np.sum(dv[:, :, h] * v[:, :, h]) - np.sum(do[:, :, h] * o[:, :, h])) < 1e-10


def pin_ring_backward(orc):
    """Backward ring: per-shard contributions under the final (O, lse) sum to torch.autograd's
    gradients through SDPA (CPU float64) over all keys; a shard wholly in the future adds zero."""
    import torch
    import torch.nn.functional as F
    rng = _rng(23)
    B, Lq, H, D = 1, 40, 2, 8
    n_shards, shard = 6, 24
    Lk = n_shards * shard
    q_off = 3 * shard + 5
    q, do = _rand(rng, B, Lq, H, D), _rand(rng, B, Lq, H, D)
    k, v = _rand(rng, B, Lk, H, D), _rand(rng, B, Lk, H, D)
    ids = np.repeat(np.arange(5), [30, 17, 41, 9, 47])[None, :]     # packed row, global coordinates
    seg_q, seg_k = ids[:, q_off:q_off + Lq], ids[:, :Lk]
    gq = np.arange(Lq) + q_off
    mask = (np.arange(Lk)[None, :] <= gq[:, None]) & (seg_q[0][:, None] == seg_k[0][None, :])
    assert mask.any(axis=1).all()
    tq, tk, tv = (torch.tensor(np.transpose(a, (0, 2, 1, 3)), requires_grad=True) for a in (q, k, v))
    tmask = torch.from_numpy(mask)[None, None]
    out = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=tmask)
    out.backward(torch.from_numpy(np.ascontiguousarray(np.transpose(do, (0, 2, 1, 3)))))
    scores = (tq.detach() @ tk.detach().transpose(-1, -2)) / math.sqrt(D)
    lse = torch.logsumexp(scores.masked_fill(~tmask, -math.inf), dim=-1).numpy()       # [B, H, Lq]
    o = np.transpose(out.detach().numpy(), (0, 2, 1, 3))
    ref_dq, ref_dk, ref_dv = (np.transpose(t.grad.numpy(), (0, 2, 1, 3)) for t in (tq, tk, tv))
    dq_sum = np.zeros_like(q)
    for j in (3, 2, 1, 0, 5, 4):                                     # ring order from the home shard
        sl = slice(j * shard, (j + 1) * shard)
        dq_j, dk_j, dv_j = orc.ring_step_bwd(q, k[:, sl], v[:, sl], o, lse, do, seg_q, seg_k[:, sl],
                                             q_off, j * shard, True, None, threads=1)
        dq_sum += dq_j
        assert np.allclose(dk_j, ref_dk[:, sl], atol=1e-11, rtol=0), j
        assert np.allclose(dv_j, ref_dv[:, sl], atol=1e-11, rtol=0), j
        if j == 5:                                                   # keys 120.. are all in the future
            assert not np.any(dq_j) and not np.any(dk_j) and not np.any(dv_j)
    assert np.allclose(dq_sum, ref_dq, atol=1e-11, rtol=0)


def pin_training_step_autograd(orc):
    """Gradients w.r.t. pre-RoPE Q, K: RoPE as complex multiplication + SDPA under autograd."""
    import torch
    import torch.nn.functional as F
    rng = _rng(21)
    B, L, H, D, theta = 1, 33, 2, 8, 1.0e4
    q, k, v, do = (_rand(rng, B, L, H, D) for _ in range(4))
    seg = np.repeat(np.arange(3), [10, 13, 10])[None, :]
    pos = orc.segment_positions(seg)
    ang = torch.tensor(pos[..., None] * (theta ** (-(2.0 * np.arange(D // 2)) / D)))  # [B, L, D/2]
    rot = torch.polar(torch.ones_like(ang), ang)[:, :, None, :]

    def rope_t(x):  # half layout: z = x_i + 1j x_{i+D/2}
        z = torch.complex(x[..., : D // 2], x[..., D // 2:]) * rot
        return torch.cat([z.real, z.imag], dim=-1)

    tq, tk, tv = (torch.tensor(a, requires_grad=True) for a in (q, k, v))
    mask = torch.from_numpy(np.tril(np.ones((L, L), dtype=bool))[None] & (seg[:, :, None] == seg[:, None, :]))
    perm = lambda x: x.permute(0, 2, 1, 3)
    out = F.scaled_dot_product_attention(perm(rope_t(tq)), perm(rope_t(tk)), perm(tv), attn_mask=mask[:, None])
    out.backward(perm(torch.tensor(do)))
    o, lse, dq, dk, dv = orc.training_step(q, k, v, do, pos, pos, theta, "half", seg, seg, threads=1)
    assert np.allclose(o, perm(out).detach().numpy(), atol=1e-12, rtol=0)
    for g, t in ((dq, tq), (dk, tk), (dv, tv)):
        assert np.allclose(g, t.grad.numpy(), atol=1e-11, rtol=0)


# ---------------------------------------------------------------- golden worked examples
def pin_golden(orc):
    with open(os.path.join(GOLDEN, "worked_attention.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        q = np.array(c["q"], dtype=np.float64)[None, :, None, :]
        k = np.array(c["k"], dtype=np.float64)[None, :, None, :]
        v = np.array(c["v"], dtype=np.float64)[None, :, None, :]
        seg = None if c.get("seg") is None else np.array(c["seg"])[None, :]
        o, lse = orc.attention_fwd(q, k, v, seg, seg, 0, 0, True, c.get("scale"), threads=1)
        assert np.allclose(o[0, :, 0, :], np.array(c["o"]), atol=1e-12, rtol=0), c["name"]
        assert np.allclose(lse[0, 0], np.array(c["lse"]), atol=1e-12, rtol=0), c["name"]
    with open(os.path.join(GOLDEN, "worked_rope.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        x = np.array(c["x"], dtype=np.float64)[None, None, None, :]
        y = orc.rope(x, [c["pos"]], c["theta"], c["layout"], inverse=c.get("inverse", False))
        assert np.allclose(y[0, 0, 0], np.array(c["y"]), atol=1e-14, rtol=0), c["name"]


# ---------------------------------------------------------------- feed-forward pins
def _ffn_case(seed, M=13, d=12, f=20):
    rng = _rng(seed, 7)
    return (_rand(rng, M, d), _rand(rng, f, d) / math.sqrt(d), _rand(rng, f, d) / math.sqrt(d),
            _rand(rng, d, f) / math.sqrt(f))


def pin_ffn_brute_force(orc):
    """Scalar loops with math.exp for z / (1 + e^-z)."""
    x, wg, wu, wd = _ffn_case(30, M=5, d=6, f=7)
    y, h = orc.swiglu_ffn(x, wg, wu, wd)
    for m in range(5):
        hh = []
        for n in range(7):
            g = math.fsum(x[m, k] * wg[n, k] for k in range(6))
            u = math.fsum(x[m, k] * wu[n, k] for k in range(6))
            hh.append(g / (1.0 + math.exp(-g)) * u)
            assert abs(h[m, n] - hh[-1]) < 1e-13
        for j in range(6):
            assert abs(y[m, j] - math.fsum(hh[n] * wd[j, n] for n in range(7))) < 1e-12


def pin_ffn_torch(orc):
    """Library routine: torch.nn.functional.silu and matmul (CPU float64), the LLaMA block."""
    import torch
    import torch.nn.functional as F
    x, wg, wu, wd = _ffn_case(31, M=40, d=32, f=88)
    t = [torch.from_numpy(a) for a in (x, wg, wu, wd)]
    ref = (F.silu(t[0] @ t[1].T) * (t[0] @ t[2].T)) @ t[3].T
    assert np.allclose(orc.swiglu_ffn(x, wg, wu, wd)[0], ref.numpy(), atol=1e-12, rtol=0)


def pin_silu_identities(orc):
    z = np.concatenate([np.linspace(-40, 40, 801), [0.0, 1e-300, -1e-300, 700.0, -700.0]])
    s = orc.silu(z)
    assert np.allclose(s - orc.silu(-z), z, atol=1e-12, rtol=1e-15)   # z sig(z) + z sig(-z) = z
    assert s[np.argmin(np.abs(z))] == 0.0 and np.isfinite(s).all()
    assert abs(orc.silu(700.0) - 700.0) < 1e-9 and abs(orc.silu(-700.0)) < 1e-9
    assert abs(orc.silu(1.0) - 1.0 / (1.0 + math.exp(-1.0))) < 1e-15


def pin_ffn_blockwise_invariance(orc):
    """Chunking the token axis (scan_mlp_chunk_size) leaves the result unchanged."""
    x, wg, wu, wd = _ffn_case(32, M=29, d=16, f=24)
    full = orc.swiglu_ffn(x, wg, wu, wd)[0]
    for chunk in (1, 3, 7, 8, 29, 64):
        assert np.allclose(orc.blockwise_ffn(x, wg, wu, wd, chunk), full, atol=1e-13, rtol=0), chunk


FFN_PINS = [pin_ffn_brute_force, pin_ffn_torch, pin_silu_identities, pin_ffn_blockwise_invariance]

ALL_PINS = [
    pin_forward_brute_force, pin_forward_sdpa, pin_forward_closed_forms, pin_forward_invariants,
    pin_packed_equals_unpacked, pin_block_and_ring_invariance, pin_rope, pin_segment_positions,
    pin_backward_finite_differences, pin_backward_autograd, pin_backward_identities,
    pin_training_step_autograd, pin_ring_backward, pin_golden,
]
