#!/usr/bin/env python3
"""Attention fwd+bwd throughput on one MI355X, as one JSON line.

A step is one pass of the whole path over one batch of synthetic input that
is already resident in HBM: attn_fwd (O, lse) then attn_bwd (dQ, dK, dV),
both through the C ABI of libattn.so.  The default workload is causal
attention with B=4, H=32, N=4096, d=128 in bf16.  Throughput counts
4*B*H*N^2*d flops for the forward (halved when causal) and 2.5x that for the
backward.

Besides the headline number the line carries:
  roofline      the dominant kernel's counted flops per launch over its
                average duration, both measured live with HIP events that
                the launches themselves record, against MI355X's dense
                bf16/fp16 MFMA peak;
  cpu_baseline  the fp64 oracle timed on this host on a bounded sample of
                the same workload (whole heads, until ~15 s of CPU work).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402

METRIC = "attention fwd+bwd TFLOP/s at d=128, N=4096 causal; % of bf16 MFMA peak"
PEAK_TFLOPS = 2516.6   # MI355X dense bf16/fp16 MFMA: 256 CU x 4096 flop/clk x 2.4 GHz
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
KERNEL_SOURCES = {
    "fwd": "exact_attention_66_amd/csrc/attn_fwd.hip",
    "bwd_dkdv": "exact_attention_66_amd/csrc/attn_bwd.hip",
    "bwd_dq": "exact_attention_66_amd/csrc/attn_bwd.hip",
}


def source_hash(kernel: str) -> str | None:
    path = KERNEL_SOURCES.get(kernel)
    if path is None:
        return None
    files = [path, "exact_attention_66_amd/csrc/attn_device.h"]
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source; otherwise None."""
    try:
        with open(TRAFFIC_FILE) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    rec = data.get(workload, {}).get(kernel)
    if not rec or rec.get("source_hash") != source_hash(kernel):
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(w: workloads.Workload, x, budget_s: float):
    """Time the fp64 oracle (as it stands) on whole heads of the workload."""
    import numpy as np
    import oracle

    heads, flops, t0 = 0, 0.0, time.perf_counter()
    per_head_fwd = w.fwd_flops() / (w.B * w.H)
    per_head = per_head_fwd + (w.bwd_flops() / (w.B * w.H) if w.backward else 0.0)
    rb = 2048 if w.N > 4096 else None
    for b in range(w.B):
        for h in range(w.H):
            q, k, v = (workloads.to_f64_numpy(x[n][b, h]) for n in ("q", "k", "v"))
            oracle.forward_head(q, k, v, w.scale, w.causal, row_block=rb)
            if w.backward:
                oracle.backward_head(q, k, v, workloads.to_f64_numpy(x["do"][b, h]), w.scale, w.causal,
                                     row_block=rb)
            heads += 1
            flops += per_head
            if time.perf_counter() - t0 >= budget_s:
                break
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    threads = None
    try:
        import threadpoolctl
        info = [i for i in threadpoolctl.threadpool_info() if i.get("user_api") == "blas"]
        threads = max((i.get("num_threads") or 0) for i in info) if info else None
    except Exception:
        threads = None
    return {
        "value": round(flops / dt / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": threads or os.cpu_count(),
        "kind": "oracle",
        "sample": (f"{heads} of {w.B * w.H} heads (b, h in order) of {w.name}, "
                   f"{'fwd+bwd' if w.backward else 'fwd'}, numpy fp64, {dt:.1f} s"),
        "host_cpus": os.cpu_count(),
        "seconds": round(dt, 2),
    }


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=workloads.HEADLINE, choices=sorted(workloads.WORKLOADS))
    ap.add_argument("--cpu-baseline-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration-bytes", type=int, default=0,
                    help="after the timed steps, also run a plain device copy of this many bytes "
                         "(reference kernel for scaling the HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); this library has no "
              "multi-GPU path: run with --gpus 1", file=sys.stderr)
        return 2

    import torch
    import exact_attention_66_amd as ea

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    ea.load()

    w = workloads.WORKLOADS[args.workload]
    x = workloads.make_inputs(w)
    dev = torch.device("cuda:0")
    q, k, v = (x[n].to(dev) for n in ("q", "k", "v"))
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    if w.backward:
        do = x["do"].to(dev)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
        ws = torch.empty(ea.attn_bwd_workspace_bytes(*w.shape()), dtype=torch.uint8, device=dev)

    def step():
        ea.attn_fwd(q, k, v, o, lse, w.scale, w.causal)
        if w.backward:
            ea.attn_bwd(q, k, v, o, do, lse, dq, dk, dv, w.scale, w.causal, ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ea.attn_profile_start()
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    prof = ea.attn_profile_stop()
    ms_per_step = e0.elapsed_time(e1) / args.steps

    if args.copy_calibration_bytes:
        src = torch.empty(args.copy_calibration_bytes, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    flops = w.fwd_flops() + w.bwd_flops()
    value = flops / (ms_per_step * 1e-3) / 1e12

    # algorithmic (counted) flops each kernel carries: the backward's five
    # products are S, dP, dV, dK (in bwd_dkdv) and dQ (in bwd_dq, which also
    # recomputes S and dP: extra work that is not counted)
    flops_per_launch = {"fwd": w.fwd_flops(), "bwd_dkdv": 0.8 * w.bwd_flops(), "bwd_dq": 0.2 * w.bwd_flops()}
    kernels = {kname: {"launches": n, "avg_ms": round(t / n, 5)} for kname, (n, t) in prof.items() if n}
    dominant = max((kname for kname in kernels if kname in flops_per_launch),
                   key=lambda kname: prof[kname][1])
    avg_ms = prof[dominant][1] / prof[dominant][0]
    achieved = flops_per_launch[dominant] / (avg_ms * 1e-3) / 1e12
    roofline = {
        "kernel": dominant,
        "bound": "mfma",
        "achieved": round(achieved, 2),
        "peak": PEAK_TFLOPS,
        "unit": "TFLOP/s",
        "frac": round(achieved / PEAK_TFLOPS, 4),
        "traffic": measured_traffic(dominant, w.name),
    }

    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "causal": w.causal,
                   "passes": "fwd+bwd" if w.backward else "fwd", "seed": w.seed},
        "pct_of_peak": round(100 * value / PEAK_TFLOPS, 2),
        "kernels": kernels,
        "roofline": roofline,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, x, args.cpu_baseline_seconds)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
