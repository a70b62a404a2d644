#!/usr/bin/env python3
"""Benchmark of the hot path on one MI355X: prints ONE JSON line.

A step is one training step of the LLaMA-7B-shaped attention layer at L = 32768 (B=1, 32 heads,
D=128, bf16, theta = 1e6, causal): RoPE on Q and K, blockwise attention forward (saving lse),
backward (delta, dQ, dK/dV) and inverse RoPE of dQ and dK, all through the C ABI.  Inputs are
seeded N(0,1) and resident in HBM before the timed region.  ``value`` is algorithmic
causal-attention TFLOP/s of forward + backward (visible pairs only, 4*D + 10*D flop per pair).

Also reported: per-kernel durations from HIP events recorded around every launch on its
stream during the timed steps, the roofline of the dominant kernel, what the matrix cores
sustain on this machine with nothing else in the loop (random N(0,1) and constant operands), the CPU
oracle timed on a bounded sample of the same workload, and (unless --no-extras) the
forward-only, packed, ring and feed-forward workloads as extra lines inside the same JSON object.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "causal attention TFLOP/s fwd+bwd and % of bf16 MFMA peak at L=32K; tokens/s"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_work(w, name):
    """Algorithmic (flop, bytes) of one launch of `name` on workload w."""
    pairs, D = w.visible_pairs(), w.D
    t = w.tensor_bytes()
    lse_bytes = 4 * w.B * w.H * w.Lq
    table = {
        "attn_fwd_bf16": (4 * D * pairs, w.fwd_bytes()),
        "attn_fwd_f32": (4 * D * pairs, w.fwd_bytes()),
        # fused RoPE: reads pre-RoPE Q, also writes the rotated Q
        "attn_fwd_rope_bf16": (4 * D * pairs, w.fwd_bytes() + t),
        # the dK/dV kernel forms S, dP, dV and dK: four of the backward's five products
        "bwd_dkdv": (8 * D * pairs, 6 * t),
        # the dQ kernel's share of the method's products is dQ (its S and dP are recomputation)
        "bwd_dq": (2 * D * pairs, 5 * t + 2 * lse_bytes),
        # dQ from the stored dS: reads two bytes of dS per visible pair and K, writes dQ
        "bwd_dq_ds": (2 * D * pairs, 2 * pairs + 2 * t),
        "bwd_delta": (0, 2 * t + lse_bytes),
        "rope_bf16": (0, 2 * t),
        "rope_f32": (0, 2 * t),
    }
    return table.get(name, (0, 0))


def time_steps(step, steps, warmup, lwm, torch):
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    lwm.lwm_profile_reset()
    lwm.lwm_profile_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    lwm.lwm_profile_enable(False)
    prof = lwm.lwm_profile_read()
    return (t1 - t0) * 1e3 / steps, prof


def time_settled(step, steps, warmup, lwm, torch, warm_ms=300.0, timed_ms=600.0):
    """time_steps with the warm-up and the timed steps raised until they cover about warm_ms and
    timed_ms of work: the extra workloads follow seconds of host-side input generation, after which
    the GPU clock takes a while under load to settle (a few short steps time it low).  Returns
    (ms per step, profile, timed steps, warm-up steps)."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    step()
    torch.cuda.synchronize()
    one = max((time.perf_counter() - t0) * 1e3, 1e-3)
    w = max(warmup, math.ceil(warm_ms / one))
    k = max(steps, math.ceil(timed_ms / one))
    ms, prof = time_steps(step, k, w, lwm, torch)
    return ms, prof, k, w


def mfma_ceiling(torch, lwm, configs, blocks=512, iters=131072):
    """What the bf16 matrix cores sustain on this machine with nothing else in the loop
    (lwm_probe_mfma_bf16: 4 independent 32x32x16 MFMA chains per wave, one wave per SIMD,
    operands in registers), for N(0,1) operands like the attention's Q, K, V and dO, and for a
    constant operand.  The chip holds a lower clock under its power limit when more operand bits
    toggle, so this, not the rated peak, is the most any kernel on these inputs can reach."""
    out = {"unit": "TFLOP/s", "peak": configs.PEAK_BF16_TFLOPS, "blocks": blocks, "iters": iters}
    n = blocks * 256 * 128
    g = torch.Generator(device="cuda").manual_seed(20261203)
    sink = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    flop = blocks * 4 * iters * 4 * 32768
    for name, src in (("random_normal", torch.randn(n, generator=g, device="cuda").to(torch.bfloat16)),
                      ("constant", torch.full((n,), 0.01, device="cuda", dtype=torch.bfloat16))):
        _, prof, k, wu = time_settled(lambda: lwm.lwm_probe_mfma_bf16(src, iters, sink), 3, 1, lwm, torch)
        total_ms, launches = prof["mfma_probe"]
        out[name] = flop / (total_ms / launches * 1e-3) / 1e12
        out[name + "_frac"] = out[name] / configs.PEAK_BF16_TFLOPS
        out[name + "_launches"] = launches
    return out


def kernels_table(prof, steps):
    return {k: {"avg_ms": ms / n, "launches_per_step": n / steps, "ms_per_step": ms / steps}
            for k, (ms, n) in sorted(prof.items(), key=lambda kv: -kv[1][0])}


def roofline_for(w, kernels, configs, traffic=None):
    name = max(kernels, key=lambda k: kernels[k]["ms_per_step"])
    flop, nbytes = kernel_work(w, name)
    avg_s = kernels[name]["avg_ms"] * 1e-3
    if flop:
        achieved = flop / avg_s / 1e12
        out = {"kernel": name, "bound": "mfma", "achieved": achieved, "peak": configs.PEAK_BF16_TFLOPS,
               "unit": "TFLOP/s", "frac": achieved / configs.PEAK_BF16_TFLOPS}
    else:
        achieved = nbytes / avg_s / 1e9
        out = {"kernel": name, "bound": "hbm", "achieved": achieved, "peak": configs.PEAK_HBM_GBS,
               "unit": "GB/s", "frac": achieved / configs.PEAK_HBM_GBS}
    out["traffic"] = (traffic or {}).get(name)
    out["avg_ms"] = kernels[name]["avg_ms"]
    return out


def load_traffic(w):
    """HBM bytes per launch measured with rocprofv3 counters (profiles/traffic_<workload>.json)."""
    p = os.path.join(ROOT, "profiles", f"traffic_{w.name}.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        rec = json.load(f)
    from ring_causal_attention_amd import build
    if rec.get("sources_sha") != build.sources_digest(rec.get("sources_family")):
        return None  # kernels changed since the counters were taken
    return {k: v["bytes_per_launch"] for k, v in rec.get("kernels", {}).items()}


def cpu_baseline(w, h, theta, heads=1):
    """The oracle (float64 numpy) on a bounded sample: `heads` heads of the same training step."""
    import numpy as np
    import oracle
    from ring_causal_attention_amd.synth import round_to_bf16
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    sl = lambda x: round_to_bf16(x[:, :, :heads]).astype(np.float64)
    pos = oracle.positions(w.B, w.Lq)
    q, k, v, do = sl(h["q"]), sl(h["k"]), sl(h["v"]), sl(h["do"])
    t0 = time.perf_counter()
    oracle.training_step(q, k, v, do, pos, pos, theta, "half", threads=threads)
    dt = time.perf_counter() - t0
    flop = (w.total_flop() // w.H) * heads
    return {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{heads} of {w.H} heads of the L={w.Lq} training step (RoPE, forward, backward, "
                      f"inverse RoPE), float64 numpy, {dt:.1f} s"}


def bench_extras(torch, lwm, path, workloads, configs, steps=3, warmup=1):
    out = {}
    W = configs.WORKLOADS
    # forward only at L = 32768 (RoPE on Q, K + forward)
    w = W["llama7b_fwd_L32768"]
    d = workloads.device_inputs(workloads.host_inputs(w))
    qr, kr = torch.empty_like(d["q"]), torch.empty_like(d["k"])
    o = torch.empty_like(d["q"])
    lse = torch.empty((w.B, w.H, w.Lq), dtype=torch.float32, device="cuda")

    def fwd_step():
        lwm.lwm_rope_apply(d["q"], qr, theta=w.theta)
        lwm.lwm_rope_apply(d["k"], kr, theta=w.theta)
        lwm.lwm_blockattn_fwd(qr, kr, d["v"], o=o, lse=lse)

    ms, prof, n, nw = time_settled(fwd_step, steps, warmup, lwm, torch)
    ks = kernels_table(prof, n)
    fk = ks["attn_fwd_bf16"]["avg_ms"]
    out[w.name] = {"ms_per_step": ms, "tflops_with_rope": w.fwd_flop() / ms / 1e9,
                   "attn_fwd_ms": fk, "attn_fwd_tflops": w.fwd_flop() / fk / 1e9,
                   "pct_of_bf16_peak": 100 * w.fwd_flop() / fk / 1e9 / configs.PEAK_BF16_TFLOPS,
                   "tokens_per_s": w.B * w.Lq / (ms * 1e-3), "steps": n, "warmup": nw, "kernels": ks}
    del d, qr, kr, o, lse
    torch.cuda.empty_cache()

    # packed row of 65536 tokens, block-diagonal causal mask
    w = W["packed_L65536"]
    d = workloads.device_inputs(workloads.host_inputs(w))
    qr, kr, o = torch.empty_like(d["q"]), torch.empty_like(d["k"]), torch.empty_like(d["q"])
    lse = torch.empty((w.B, w.H, w.Lq), dtype=torch.float32, device="cuda")

    def packed_step():
        lwm.lwm_rope_apply(d["q"], qr, seg=d["seg"], theta=w.theta)
        lwm.lwm_rope_apply(d["k"], kr, seg=d["seg"], theta=w.theta)
        lwm.lwm_blockattn_fwd(qr, kr, d["v"], d["seg"], d["seg"], o=o, lse=lse)

    ms, prof, n, nw = time_settled(packed_step, steps, warmup, lwm, torch)
    ks = kernels_table(prof, n)
    fk = ks["attn_fwd_bf16"]["avg_ms"]
    out[w.name] = {"ms_per_step": ms, "attn_fwd_ms": fk, "attn_fwd_tflops": w.fwd_flop() / fk / 1e9,
                   "pct_of_bf16_peak": 100 * w.fwd_flop() / fk / 1e9 / configs.PEAK_BF16_TFLOPS,
                   "segments": len(w.segment_lengths()), "visible_pairs": w.visible_pairs(), "steps": n, "warmup": nw, "kernels": ks}
    # the same packed row through a whole training step (forward + backward, segment-aware tile
    # skipping in both backward kernels); dO drawn like the other tensors of the workload
    from ring_causal_attention_amd import synth
    do = workloads.to_device(synth.normal(w.seed, "do", (w.B, w.Lq, w.H, w.D)), w.dtype)
    bufs = path.TrainStepBuffers(d["q"], d["k"])

    def packed_train_step():
        path.training_step(d["q"], d["k"], d["v"], do, w.theta, seg=d["seg"], buffers=bufs)

    ms, prof, n, nw = time_settled(packed_train_step, steps, warmup, lwm, torch)
    ks = kernels_table(prof, n)
    tflop = 14 * w.D * w.visible_pairs()
    bk = sum(ks[k]["ms_per_step"] for k in ("bwd_delta", "bwd_dq", "bwd_dq_ds", "bwd_dkdv") if k in ks)
    out[w.name + "_train"] = {"ms_per_step": ms, "tflops": tflop / ms / 1e9,
                              "pct_of_bf16_peak": 100 * tflop / ms / 1e9 / configs.PEAK_BF16_TFLOPS,
                              "attn_bwd_ms": bk, "attn_bwd_tflops": 10 * w.D * w.visible_pairs() / bk / 1e9,
                              "tokens_per_s": w.B * w.Lq / (ms * 1e-3), "steps": n, "warmup": nw, "kernels": ks}

    # the same step through the fused-RoPE calls (positions restart per segment inside the kernels)
    def packed_train_step_fused():
        path.training_step_fused(d["q"], d["k"], d["v"], do, w.theta, seg=d["seg"], buffers=bufs)

    ms, prof, n, nw = time_settled(packed_train_step_fused, steps, warmup, lwm, torch)
    ks = kernels_table(prof, n)
    out[w.name + "_train"]["rope_fused"] = {
        "ms_per_step": ms, "tflops": tflop / ms / 1e9, "pct_of_bf16_peak": 100 * tflop / ms / 1e9 / configs.PEAK_BF16_TFLOPS,
        "tokens_per_s": w.B * w.Lq / (ms * 1e-3), "steps": n, "warmup": nw, "kernels": ks,
        "note": "same workload and flop count; one RoPE pass (K) instead of four"}
    del d, qr, kr, o, lse, do, bufs
    torch.cuda.empty_cache()

    # one device's share of a 1M-token ring: 41 visible shards folded by lwm_ring_step
    w = W["ring_share_1M"]
    d = workloads.device_inputs(workloads.host_inputs(w))
    S = w.Lq
    qr = lwm.lwm_rope_apply(d["q"], pos_offset=w.q_offset, theta=w.theta)
    kr = {j: lwm.lwm_rope_apply(x, pos_offset=j * S, theta=w.theta) for j, x in d["k_shards"].items()}
    o_acc = torch.empty((w.B, S, w.H, w.D), dtype=torch.float32, device="cuda")
    lse_acc = torch.empty((w.B, w.H, S), dtype=torch.float32, device="cuda")
    o = torch.empty_like(qr)

    def ring_step():
        o_acc.zero_()
        lse_acc.fill_(float("-inf"))
        path.ring_forward(qr, kr, d["v_shards"], w.ring_order(), S, w.q_offset, o_acc=o_acc, lse_acc=lse_acc,
                          o_final=o)

    ms, prof, n, nw = time_settled(ring_step, steps, warmup, lwm, torch)
    ks = kernels_table(prof, n)
    rk = ks["ring_step_bf16"]
    out[w.name] = {"ms_per_step": ms, "ring_steps_per_pass": rk["launches_per_step"],
                   "ring_kernel_ms_per_pass": rk["ms_per_step"],
                   "tflops": w.fwd_flop() / ms / 1e9,
                   "ring_kernel_tflops": w.fwd_flop() / rk["ms_per_step"] / 1e9,
                   "pct_of_bf16_peak": 100 * w.fwd_flop() / rk["ms_per_step"] / 1e9 / configs.PEAK_BF16_TFLOPS,
                   "query_tokens_per_s": w.B * S / (ms * 1e-3), "steps": n, "warmup": nw, "kernels": ks}

    # the same share's backward ring: the 41 shards visit again, each adding its share of the
    # gradients (dQ stays, dK / dV travel with their shard); o / lse_acc hold the forward's result
    f32 = dict(dtype=torch.float32, device="cuda")
    dq_acc = torch.empty((w.B, S, w.H, w.D), **f32)
    dk_acc = {j: torch.empty((w.B, S, w.H, w.D), **f32) for j in kr}
    dv_acc = {j: torch.empty((w.B, S, w.H, w.D), **f32) for j in kr}
    ws = lwm.bwd_workspace(w.B, w.H, S, S, w.D, "cuda", causal=False)  # dense: every shard offset

    def ring_bwd_step():
        for t in (dq_acc, *dk_acc.values(), *dv_acc.values()):
            t.zero_()
        path.ring_backward(qr, kr, d["v_shards"], o, lse_acc, d["do"], w.ring_order(), S, w.q_offset,
                           dq_acc=dq_acc, dk_acc=dk_acc, dv_acc=dv_acc, workspace=ws)

    ms, prof, n, nw = time_settled(ring_bwd_step, steps, warmup, lwm, torch)
    ks = kernels_table(prof, n)
    kms = sum(ks[k]["ms_per_step"] for k in ("bwd_delta", "bwd_dq", "bwd_dq_ds", "bwd_dkdv") if k in ks)
    bflop = 10 * w.D * w.visible_pairs()
    out[w.name + "_backward"] = {
        "ms_per_step": ms, "ring_steps_per_pass": ks["bwd_dkdv"]["launches_per_step"],
        "kernel_ms_per_pass": kms, "tflops": bflop / ms / 1e9, "kernel_tflops": bflop / kms / 1e9,
        "pct_of_bf16_peak": 100 * bflop / kms / 1e9 / configs.PEAK_BF16_TFLOPS,
        "note": "10*D flop per visible pair; ms_per_step also zeroes the float32 accumulators",
        "steps": n, "warmup": nw, "kernels": ks}
    del d, qr, kr, o_acc, lse_acc, o, dq_acc, dk_acc, dv_acc, ws
    torch.cuda.empty_cache()

    # the blockwise feed-forward block that follows the attention (LLaMA-7B SwiGLU, chunks of
    # 8192 rows), timed beside the same three products through torch.matmul (hipBLASLt)
    fw = configs.FFN_WORKLOADS["ffn_llama7b_L32768"]
    from ring_causal_attention_amd import synth
    hf = synth.ffn_inputs(fw.seed, fw.rows, fw.d_model, fw.d_ff)
    df = {k: workloads.to_device(v, "bf16") for k, v in hf.items()}
    del hf
    y = torch.empty_like(df["x"])
    fws = torch.empty(lwm.lwm_blockwise_ffn_workspace_size(fw.rows, fw.d_ff, fw.chunk), dtype=torch.uint8,
                      device="cuda")

    def ffn_step():
        lwm.lwm_blockwise_ffn(df["x"], df["w_gate"], df["w_up"], df["w_down"], chunk=fw.chunk, y=y, workspace=fws)

    ms, prof, n, nw = time_settled(ffn_step, steps, warmup, lwm, torch)
    ks = kernels_table(prof, n)
    per_chunk = 2 * fw.chunk * fw.d_model * fw.d_ff
    traffic = load_traffic(fw) or {}
    roof = {}
    for name, mult in (("ffn_gate_up", 2), ("ffn_down", 1)):
        if name in ks:
            ach = mult * per_chunk / (ks[name]["avg_ms"] * 1e-3) / 1e12
            roof[name] = {"bound": "mfma", "achieved": ach, "peak": configs.PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                          "frac": ach / configs.PEAK_BF16_TFLOPS, "traffic": traffic.get(name),
                          "avg_ms": ks[name]["avg_ms"]}
    wg, wu, wd = df["w_gate"], df["w_up"], df["w_down"]

    def torch_step():
        for r0 in range(0, fw.rows, fw.chunk):
            xc = df["x"][r0:r0 + fw.chunk]
            torch.matmul(torch.nn.functional.silu(torch.matmul(xc, wg.t())) * torch.matmul(xc, wu.t()), wd.t(),
                         out=y[r0:r0 + fw.chunk])

    for _ in range(nw):
        torch_step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(n):
        torch_step()
    torch.cuda.synchronize()
    torch_ms = (time.perf_counter() - t0) * 1e3 / n
    out[fw.name] = {"ms_per_step": ms, "tflops": fw.flop() / ms / 1e9,
                    "pct_of_bf16_peak": 100 * fw.flop() / ms / 1e9 / configs.PEAK_BF16_TFLOPS,
                    "tokens_per_s": fw.rows / (ms * 1e-3), "roofline": roof,
                    "torch_matmul_ms_per_step": torch_ms,
                    "note": "6*rows*d_model*d_ff flop; torch_matmul_ms_per_step runs the same three products "
                            "through torch.matmul and silu for comparison", "steps": n, "warmup": nw, "kernels": ks}
    del df, y, fws
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-extras", action="store_true", help="skip the forward / packed / ring lines")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=1, help="heads of the oracle sample")
    ap.add_argument("--no-mfma-ceiling", action="store_true", help="skip the matrix-core rate probe")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE={world}).  The ring is simulated on one GPU as a loop over KV shards.", file=sys.stderr)
        sys.exit(2)

    import torch
    from ring_causal_attention_amd import configs, lwm, path, workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    lwm.lib()  # fail loudly if the HIP library is missing
    w = configs.WORKLOADS["train_step_L32768"]
    log(f"[bench] generating {w.name} inputs")
    h = workloads.host_inputs(w)
    d = workloads.device_inputs(h)
    bufs = path.TrainStepBuffers(d["q"], d["k"])

    def step():
        path.training_step(d["q"], d["k"], d["v"], d["do"], w.theta, buffers=bufs)

    log(f"[bench] timing {args.steps} steps after {args.warmup} warm-up steps")
    ms, prof = time_steps(step, args.steps, args.warmup, lwm, torch)
    kernels = kernels_table(prof, args.steps)
    flop = w.total_flop()
    value = flop / (ms * 1e-3) / 1e12
    fk = kernels["attn_fwd_bf16"]
    bwd_ms = sum(kernels[k]["ms_per_step"] for k in ("bwd_delta", "bwd_dq", "bwd_dq_ds", "bwd_dkdv") if k in kernels)
    result = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.B, "seq_len": w.Lq, "heads": w.H, "head_dim": w.D,
                   "theta": w.theta, "causal": True, "rope_layout": "half", "fwd_tile": "128 queries x 64 keys",
                   "bwd_tiles": "dK/dV: 256 keys x 64 queries, storing dS; dQ from stored dS: 256 queries x 64 keys",
                   "bwd_ds_heads_per_pass": lwm.default_ds_heads(w.B, w.H, w.Lq, w.Lk, w.D)},
        "pct_of_bf16_peak": 100 * value / configs.PEAK_BF16_TFLOPS,
        "tokens_per_s": w.B * w.Lq / (ms * 1e-3),
        "attention_fwd_tflops": w.fwd_flop() / fk["avg_ms"] / 1e9,
        "attention_bwd_tflops": w.bwd_flop() / bwd_ms / 1e9 if bwd_ms else None,
        "kernels": kernels,
        "roofline": roofline_for(w, kernels, configs, load_traffic(w)),
    }
    # the same step with RoPE inside the attention calls (lwm_blockattn_fwd_rope / _bwd_rope):
    # no RoPE pass over Q, no inverse-RoPE passes over dQ and dK
    def fused_step():
        path.training_step_fused(d["q"], d["k"], d["v"], d["do"], w.theta, buffers=bufs)

    log("[bench] timing the fused-RoPE training step")
    fms, fprof = time_steps(fused_step, args.steps, args.warmup, lwm, torch)
    fks = kernels_table(fprof, args.steps)
    result["train_step_rope_fused"] = {
        "ms_per_step": fms, "tflops": flop / (fms * 1e-3) / 1e12,
        "pct_of_bf16_peak": 100 * flop / (fms * 1e-3) / 1e12 / configs.PEAK_BF16_TFLOPS,
        "tokens_per_s": w.B * w.Lq / (fms * 1e-3),
        "note": "same workload and flop count as the headline step; dQ and dK rounded to bf16 once",
        "kernels": fks}
    if not args.no_mfma_ceiling:
        log("[bench] matrix-core rate probe")
        try:
            result["mfma_ceiling"] = mfma_ceiling(torch, lwm, configs)
        except (lwm.LwmError, RuntimeError) as e:  # an auxiliary figure: report it, keep the line
            log(f"[bench] matrix-core rate probe failed: {e}")
            result["mfma_ceiling"] = {"error": str(e)}
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample")
        result["cpu_baseline"] = cpu_baseline(w, h, w.theta, heads=args.cpu_heads)
    del d, bufs
    torch.cuda.empty_cache()
    if not args.no_extras:
        log("[bench] extra workloads")
        result["extra"] = bench_extras(torch, lwm, path, workloads, configs)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
