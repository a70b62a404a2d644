"""Driver for rocprofv3 runs of the hot path, and the summariser of their counter output.

``--ring-backward`` runs the backward ring of a ring workload (after one forward ring).

Run under the profiler (one counter pass per run, e.g. ``--pmc FETCH_SIZE``):

    rocprofv3 --pmc FETCH_SIZE -d OUT -o fetch -- python3 -m ring_causal_attention_amd.profile_run \
        --workload train_step_L32768 --steps 2

``--copy-mib N`` instead runs a plain device-to-device copy of N MiB (torch ``copy_``), whose
FETCH_SIZE / WRITE_SIZE give the factor that turns the counters into bytes.

``--medians`` times the attention calls of the five workloads (inputs resident in HBM, RoPE applied
beforehand) with a HIP event pair around each call on the current stream: 3 warm-up calls, then
the median, minimum and maximum of 20, printed as JSON.

``--summarize DIR`` reads the ``*_counter_collection.csv`` files under DIR and writes
``profiles/traffic_<workload>.json`` (HBM bytes per launch of each kernel, scaled by the copy
calibration, tagged with the digest of the kernel sources) plus a Markdown table on stdout.
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import sys
from collections import defaultdict

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_ffn(name: str, steps: int):
    import torch
    from . import configs, lwm, synth, workloads
    w = configs.FFN_WORKLOADS[name]
    d = {k: workloads.to_device(v, "bf16") for k, v in synth.ffn_inputs(w.seed, w.rows, w.d_model, w.d_ff).items()}
    for i in range(steps):
        lwm.lwm_blockwise_ffn(d["x"], d["w_gate"], d["w_up"], d["w_down"], chunk=w.chunk)
        torch.cuda.synchronize()
        print(f"[profile_run] {name} step {i + 1}/{steps} done", flush=True)


def run_workload(name: str, steps: int, ring_backward: bool = False):
    import torch
    from . import configs, lwm, path, workloads
    if name in configs.FFN_WORKLOADS:
        return run_ffn(name, steps)
    w = configs.WORKLOADS[name]
    d = workloads.device_inputs(workloads.host_inputs(w))
    if ring_backward:
        if not w.ring_shards:
            raise SystemExit("--ring-backward needs a ring workload")
        S = w.Lq
        qr = lwm.lwm_rope_apply(d["q"], pos_offset=w.q_offset, theta=w.theta)
        kr = {j: lwm.lwm_rope_apply(x, pos_offset=j * S, theta=w.theta) for j, x in d["k_shards"].items()}
        o, _, lse = path.ring_forward(qr, kr, d["v_shards"], w.ring_order(), S, w.q_offset)
        step = lambda: path.ring_backward(qr, kr, d["v_shards"], o, lse, d["do"], w.ring_order(), S, w.q_offset)
    elif w.backward:
        bufs = path.TrainStepBuffers(d["q"], d["k"])
        step = lambda: path.training_step(d["q"], d["k"], d["v"], d["do"], w.theta, buffers=bufs)
    elif w.ring_shards:
        S = w.Lq
        qr = lwm.lwm_rope_apply(d["q"], pos_offset=w.q_offset, theta=w.theta)
        kr = {j: lwm.lwm_rope_apply(x, pos_offset=j * S, theta=w.theta) for j, x in d["k_shards"].items()}
        step = lambda: path.ring_forward(qr, kr, d["v_shards"], w.ring_order(), S, w.q_offset)
    else:
        step = lambda: path.attention_forward(d["q"], d["k"], d["v"], w.theta, seg=d["seg"])
    for i in range(steps):
        step()
        torch.cuda.synchronize()
        print(f"[profile_run] {name} step {i + 1}/{steps} done", flush=True)


def run_copy(mib: int):
    import torch
    n = mib * (1 << 20) // 4
    x = torch.ones(n, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    print(f"[profile_run] copied {mib} MiB three times", flush=True)


def _short(kernel_name: str) -> str:
    for key in ("bwd_dkdv", "bwd_dq_ds", "bwd_dq", "bwd_delta", "attn_fwd_bf16", "attn_fwd_f32", "rope_kernel"):
        if key in kernel_name:
            return key
    if "ffn_gemm_kernel" in kernel_name:
        return "ffn_gate_up" if "ILb1E" in kernel_name or "<true" in kernel_name else "ffn_down"
    return kernel_name.split("(")[0][-60:]


def summarize(directory: str, workload: str, copy_mib: int):
    """Average per dispatch of every counter, per kernel; bytes scaled by the copy calibration."""
    vals = defaultdict(lambda: defaultdict(list))
    for f in glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for row in csv.DictReader(fh):
                k = _short(row.get("Kernel_Name", ""))
                vals[k][row["Counter_Name"]].append(float(row["Counter_Value"]))
    avg = {k: {c: sum(v) / len(v) for c, v in cs.items()} for k, cs in vals.items()}
    copy_key = next((k for k in avg if "copy" in k.lower() or "elementwise" in k.lower()), None)
    out = {"workload": workload, "counters": avg}
    if copy_key:
        nbytes = copy_mib * (1 << 20)
        fr = avg[copy_key].get("FETCH_SIZE")
        fw = avg[copy_key].get("WRITE_SIZE")
        out["calibration"] = {"copy_kernel": copy_key, "bytes": nbytes,
                              "fetch_kib_per_byte": fr / nbytes if fr else None,
                              "write_kib_per_byte": fw / nbytes if fw else None}
        kern = {}
        for k, cs in avg.items():
            if k == copy_key:
                continue
            rb = cs.get("FETCH_SIZE") / (fr / nbytes) if fr and "FETCH_SIZE" in cs else None
            wb = cs.get("WRITE_SIZE") / (fw / nbytes) if fw and "WRITE_SIZE" in cs else None
            if rb is not None or wb is not None:
                kern[k] = {"read_bytes": rb, "write_bytes": wb, "bytes_per_launch": (rb or 0) + (wb or 0)}
        out["kernels"] = kern
    from .build import sources_digest
    from .configs import FFN_WORKLOADS
    out["sources_family"] = "ffn" if workload in FFN_WORKLOADS else "attention"
    out["sources_sha"] = sources_digest(out["sources_family"])
    return out


def medians(n: int = 20, warm: int = 3) -> dict:
    """Median / min / max milliseconds of n event-timed calls per workload call (see the module doc)."""
    import statistics

    import torch

    from . import lwm, path, workloads
    from .configs import WORKLOADS

    def timed(fn):
        for _ in range(warm):
            fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(n):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            b.synchronize()
            ts.append(a.elapsed_time(b))
        return {"ms": statistics.median(ts), "min_ms": min(ts), "max_ms": max(ts), "calls": n}

    res = {}
    for name in ("causal_fp32_L1024", "llama7b_fwd_L32768", "packed_L65536", "train_step_L32768"):
        w = WORKLOADS[name]
        d = workloads.device_inputs(workloads.host_inputs(w))
        seg = d["seg"]
        qr = lwm.lwm_rope_apply(d["q"], seg=seg, theta=w.theta)
        kr = lwm.lwm_rope_apply(d["k"], seg=seg, theta=w.theta)
        o = torch.empty_like(qr)
        lse = torch.empty((w.B, w.H, w.Lq), dtype=torch.float32, device="cuda")
        r = timed(lambda: lwm.lwm_blockattn_fwd(qr, kr, d["v"], seg, seg, o=o, lse=lse))
        r["tflops"] = w.fwd_flop() / r["ms"] / 1e9
        res[name + " lwm_blockattn_fwd"] = r
        print(f"[medians] {name} forward {r['ms']:.3f} ms", flush=True)
        if w.backward:
            ws = lwm.bwd_workspace(w.B, w.H, w.Lq, w.Lk, w.D, "cuda")
            dq, dk, dv = torch.empty_like(qr), torch.empty_like(kr), torch.empty_like(d["v"])
            r = timed(lambda: lwm.lwm_blockattn_bwd(qr, kr, d["v"], o, lse, d["do"], seg, seg, dq=dq, dk=dk, dv=dv,
                                                    workspace=ws))
            r["tflops"] = w.bwd_flop() / r["ms"] / 1e9
            res[name + " lwm_blockattn_bwd"] = r
            print(f"[medians] {name} backward {r['ms']:.3f} ms", flush=True)
        del d, qr, kr, o, lse
        torch.cuda.empty_cache()
    w = WORKLOADS["ring_share_1M"]
    d = workloads.device_inputs(workloads.host_inputs(w))
    S = w.Lq
    qr = lwm.lwm_rope_apply(d["q"], pos_offset=w.q_offset, theta=w.theta)
    kr = {j: lwm.lwm_rope_apply(x, pos_offset=j * S, theta=w.theta) for j, x in d["k_shards"].items()}
    o_acc = torch.empty((w.B, S, w.H, w.D), dtype=torch.float32, device="cuda")
    lse_acc = torch.empty((w.B, w.H, S), dtype=torch.float32, device="cuda")
    o = torch.empty_like(qr)

    def ring():
        o_acc.zero_()
        lse_acc.fill_(float("-inf"))
        path.ring_forward(qr, kr, d["v_shards"], w.ring_order(), S, w.q_offset, o_acc=o_acc, lse_acc=lse_acc,
                          o_final=o)

    r = timed(ring)
    r["tflops"] = w.fwd_flop() / r["ms"] / 1e9
    res["ring_share_1M path.ring_forward (41 lwm_ring_step)"] = r
    print(f"[medians] ring_share_1M ring pass {r['ms']:.3f} ms", flush=True)
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="train_step_L32768")
    ap.add_argument("--steps", type=int, default=2)
    ap.add_argument("--copy-mib", type=int, default=0)
    ap.add_argument("--summarize", default=None)
    ap.add_argument("--write", action="store_true", help="write profiles/traffic_<workload>.json")
    ap.add_argument("--ring-backward", action="store_true", help="ring workloads: run the backward ring")
    ap.add_argument("--medians", action="store_true", help="median of 20 timed calls per workload call")
    args = ap.parse_args()
    if args.medians:
        print(json.dumps(medians(), indent=1))
        return
    if args.summarize:
        res = summarize(args.summarize, args.workload, args.copy_mib or 1024)
        if args.write:
            with open(os.path.join(ROOT, "profiles", f"traffic_{args.workload}.json"), "w") as f:
                json.dump(res, f, indent=1)
        print(json.dumps(res, indent=1))
        return
    if args.copy_mib:
        run_copy(args.copy_mib)
    else:
        run_workload(args.workload, args.steps, args.ring_backward)


if __name__ == "__main__":
    sys.exit(main())
