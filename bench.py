#!/usr/bin/env python3
"""Attention fwd+bwd throughput on one MI355X, as one JSON line.

A step is one pass of the whole path over one batch of synthetic input that
is already resident in HBM: attn_fwd (O, lse) then attn_bwd (dQ, dK, dV),
both through the C ABI of libattn.so.  The default workload is causal
attention with B=4, H=32, N=4096, d=128 in bf16.  Throughput counts
4*B*H*N^2*d flops for the forward (halved when causal) and 2.5x that for the
backward.

``value`` and ``ms_per_step`` come from the K timed steps (one event pair
around all of them, a device synchronize on both sides).  Then, per
workload:
  timing        forward and backward timed separately, each step bracketed by
                events: medians over at least 20 steps spanning at least
                0.5 s, with the GPU clock sampled meanwhile (sysfs sclk) and
                the % of peak also given against the peak at that clock;
  kernels       per-launch durations from HIP events the launches record;
  roofline      the dominant kernel's counted flops per launch over its
                average duration, against MI355X's dense bf16/fp16 MFMA peak;
  workloads     the same for every other training workload (the line's
                ``value`` stays the headline's);
  cpu_baseline  the fp64 oracle, as it stands, over whole heads of the
                headline workload in a pool of host processes (one BLAS
                thread each), within a time budget.
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

# Only the standard library at module level: the oracle pool's worker
# processes (spawn) import this file, and must not load torch or the library.

METRIC = "attention fwd+bwd TFLOP/s at d=128, N=4096 causal; % of bf16 MFMA peak"
PEAK_TFLOPS = 2516.6   # MI355X dense bf16/fp16 MFMA: 256 CU x 4096 flop/clk x 2.4 GHz
PEAK_CLOCK_MHZ = 2400.0
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
KERNEL_SOURCES = {
    "fwd": "exact_attention_66_amd/csrc/attn_fwd.hip",
    "bwd_dkdv": "exact_attention_66_amd/csrc/attn_bwd.hip",
    "bwd_dq": "exact_attention_66_amd/csrc/attn_bwd.hip",
    "kv_split": "exact_attention_66_amd/csrc/attn_kvcache.hip",
    "kv_merge": "exact_attention_66_amd/csrc/attn_kvcache.hip",
    "bwd_prep": "exact_attention_66_amd/csrc/attn_bwd.hip",
}


def source_hash(kernel: str) -> str | None:
    path = KERNEL_SOURCES.get(kernel)
    if path is None:
        return None
    files = [path, "exact_attention_66_amd/csrc/attn_device.h", "exact_attention_66_amd/csrc/attn_launch.h",
             "exact_attention_66_amd/csrc/attn_dropout.h"]
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def _code_only(text: str) -> str:
    """Source text without comments and blank lines: edits to comments do not
    invalidate a counter record taken on the same code."""
    import re
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = [re.sub(r"//.*$", "", ln).rstrip() for ln in text.splitlines()]
    return "\n".join(ln for ln in lines if ln.strip())


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


def _oracle_head(task):
    """Worker: the fp64 oracle (as it stands) on one head, forward and backward;
    returns the head's counted flops and its wall time."""
    import numpy as np
    import oracle

    q, k, v, do, scale, causal, dropout, flops = task
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    t0 = time.perf_counter()
    oracle.forward_head(q, k, v, scale, causal, row_block=512, dropout=dropout)
    if do is not None:
        oracle.backward_head(q, k, v, np.asarray(do, dtype=np.float64), scale, causal, row_block=512,
                             dropout=dropout)
    return flops, time.perf_counter() - t0


def cpu_baseline(w, x, budget_s: float, dropout=None, workers: int = 0):
    """Time the fp64 oracle (as it stands) over whole heads of the workload in a
    pool of host processes, one BLAS thread each; heads are handed out in
    (b, h) order until the time budget is spent.  ``dropout``: ``(p, seed,
    offset)`` or None."""
    import multiprocessing as mp

    workers = workers or max(1, min(16, os.cpu_count() or 1))
    per_head = (w.fwd_flops() + w.bwd_flops()) / (w.B * w.H)

    def tasks():
        for b in range(w.B):
            for h in range(w.H):
                yield (x["q"][b, h].float().numpy(), x["k"][b, h].float().numpy(), x["v"][b, h].float().numpy(),
                       x["do"][b, h].float().numpy() if w.backward else None, float(w.scale), bool(w.causal),
                       None if dropout is None else (*dropout, b * w.H + h), per_head)

    saved = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")}
    for k in saved:
        os.environ[k] = "1"
    heads, flops, busy = 0, 0.0, 0.0
    try:
        with mp.get_context("spawn").Pool(workers) as pool:
            t0 = time.perf_counter()
            for f, dt in pool.imap_unordered(_oracle_head, tasks()):
                heads += 1
                flops += f
                busy += dt
                if time.perf_counter() - t0 >= budget_s:
                    break
            wall = time.perf_counter() - t0
            pool.terminate()
    finally:
        for k, val in saved.items():
            if val is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = val
    return {
        "value": round(flops / wall / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": workers,
        "kind": "oracle",
        "sample": (f"{heads} of {w.B * w.H} heads of {w.name}, {'fwd+bwd' if w.backward else 'fwd'}, numpy fp64, "
                   f"{workers} worker processes x 1 BLAS thread, {wall:.1f} s wall ({busy:.1f} s of worker time)"),
        "host_cpus": os.cpu_count(),
        "seconds": round(wall, 2),
    }


KERNEL_NAME_KINDS = [("fwd_kernel<", "fwd"), ("bwd_prep<", "bwd_prep"), ("bwd_dkdv<", "bwd_dkdv"),
                     ("bwd_dq<", "bwd_dq"), ("kv_split_kernel<", "kv_split"), ("kv_merge_kernel<", "kv_merge")]


def record_traffic(fetch_csv: str, write_csv: str, workload: str) -> int:
    """Turn two rocprofv3 counter files (FETCH_SIZE, WRITE_SIZE; KiB per
    dispatch) of a run with --copy-calibration-bytes into HBM bytes per
    launch of each kernel: fetched and written KiB are scaled by what the same
    counters read for the plain 1 GiB device copy in that run.  Updates the
    workload's entry of profiles/hbm_traffic.json (with the current kernel
    source hash) and prints a markdown table."""
    import csv
    from collections import defaultdict

    def per_kernel(path, counter):
        vals = defaultdict(list)
        with open(path, newline="") as f:
            for row in csv.DictReader(f):
                if row.get("Counter_Name") != counter:
                    continue
                vals[row["Kernel_Name"]].append(float(row["Counter_Value"]))
        return vals

    fetch, write = per_kernel(fetch_csv, "FETCH_SIZE"), per_kernel(write_csv, "WRITE_SIZE")
    gib_kib = 1024.0 * 1024.0
    copy_f = max((max(v) for k, v in fetch.items() if "copyBuffer" in k), default=None)
    copy_w = max((max(v) for k, v in write.items() if "copyBuffer" in k), default=None)
    if not copy_f or not copy_w:
        print("no 1 GiB copy kernel in the counter files (run with --copy-calibration-bytes 1073741824)",
              file=sys.stderr)
        return 1
    fs, wsc = gib_kib / copy_f, gib_kib / copy_w
    try:
        with open(TRAFFIC_FILE) as f:
            data = json.load(f)
    except (OSError, ValueError):
        data = {}
    entry = {}
    print(f"Calibration: a plain 1 GiB device copy reads FETCH_SIZE = {copy_f:.0f} KiB and WRITE_SIZE = "
          f"{copy_w:.0f} KiB, so fetched KiB are scaled by {fs:.4f} and written KiB by {wsc:.4f}.\n")
    print("| kernel | FETCH_SIZE (KiB) | WRITE_SIZE (KiB) | scaled bytes read | scaled bytes written | total (GB) |")
    print("|---|---|---|---|---|---|")
    for name in sorted(set(fetch) & set(write)):
        kind = next((kd for pre, kd in KERNEL_NAME_KINDS if pre in name), None)
        if kind is None:
            continue
        fk = sum(fetch[name]) / len(fetch[name])
        wk = sum(write[name]) / len(write[name])
        rd, wr = fk * 1024 * fs, wk * 1024 * wsc
        entry[kind] = {"bytes_per_launch": int(rd + wr), "bytes_read": int(rd), "bytes_written": int(wr),
                       "fetch_kib": round(fk, 1), "write_kib": round(wk, 1), "fetch_scale": round(fs, 4),
                       "write_scale": round(wsc, 4), "source_hash": source_hash(kind)}
        short = name.replace("attn::(anonymous namespace)::", "").replace("void ", "").split("(")[0]
        print(f"| `{short}` | {fk:.0f} | {wk:.0f} | {rd / 1e9:.3f} GB | {wr / 1e9:.3f} GB | {(rd + wr) / 1e9:.3f} |")
    data.setdefault(workload, {}).update(entry)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(data, f, indent=1)
        f.write("\n")
    return 0


def timed_passes(step, steps: int):
    """Time `steps` steps twice, each pass bracketed by a device synchronize:
    first plainly (events around the whole pass: the step time), then with
    the library's profiling window open, in which every launch records its
    own event pair on its stream (the per-kernel durations).  Per-launch
    events add host work to each launch, about 10 us, which would otherwise
    show up as idle time between short kernels in the step time."""
    import torch
    import exact_attention_66_amd as ea

    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for i in range(steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    ms_per_step = e0.elapsed_time(e1) / steps
    ea.attn_profile_start()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    prof = ea.attn_profile_stop()
    return ms_per_step, prof


def copy_calibration(nbytes: int, dev) -> None:
    """A plain device-to-device copy of nbytes (three times): the reference
    kernel whose byte counters scale those of the attention kernels."""
    if not nbytes:
        return
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()


def cpu_baseline_kv(w: workloads.KvWorkload, x, budget_s: float):
    """Time the fp64 oracle (as it stands) on whole heads of a KV-cache workload."""
    import oracle
    import workloads

    heads, t0 = 0, time.perf_counter()
    G = w.H // w.kv_heads
    for b in range(w.B):
        for h in range(w.H):
            oracle.forward_head(workloads.to_f64_numpy(x["q"][b, h]), workloads.to_f64_numpy(x["k"][b, h // G]),
                                workloads.to_f64_numpy(x["v"][b, h // G]), w.scale, w.causal)
            heads += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    per_head = w.io_bytes() / (w.B * w.H)
    return {
        "value": round(heads * per_head / dt / 1e9, 4),
        "unit": "GB/s",
        "cores": os.cpu_count(),
        "kind": "oracle",
        "sample": f"{heads} of {w.B * w.H} heads (b, h in order) of {w.name}, numpy fp64, {dt:.2f} s",
        "host_cpus": os.cpu_count(),
        "seconds": round(dt, 3),
    }


def bench_kvcache(args, w: workloads.KvWorkload) -> int:
    """Decoding against a KV cache: one step is one attn_fwd_kvcache call
    (split kernel + merge kernel) over a batch of caches resident in HBM.
    Consecutive steps use different copies of the inputs (enough copies to
    exceed the 256 MB last-level cache three times over), so every step
    streams its K and V from HBM, as decoding a new batch would."""
    import torch
    import exact_attention_66_amd as ea
    import workloads

    dev = torch.device("cuda:0")
    x = workloads.make_kv_inputs(w)
    copies = max(1, min(8, -(-3 * 256 * 2**20 // w.kv_bytes())))
    sets = [{n: x[n].to(dev) for n in ("q", "k", "v")} for _ in range(copies)]
    o = torch.empty((w.B, w.H, w.Nq, w.d), dtype=w.torch_dtype, device=dev)
    lse = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device=dev)
    G = w.H // w.kv_heads
    if G > 1:   # grouped heads: the G query heads of a KV head share its pass over K and V
        ws = torch.empty(ea.attn_fwd_kvcache_gqa_workspace_bytes(w.B, w.H, w.kv_heads, w.Nq, w.Nk, w.d, 0),
                         dtype=torch.uint8, device=dev)
        splits = ea.attn_fwd_kvcache_splits(w.B, w.kv_heads, G * w.Nq, w.Nk, w.d, 0)
        lib = ea.load()
        stream = torch.cuda.current_stream().cuda_stream or None
        dt = ea.ATTN_DTYPE_BF16 if w.dtype == "bf16" else ea.ATTN_DTYPE_FP16

        def step(i):
            t = sets[i % copies]
            st = lib.attn_fwd_kvcache_gqa(t["q"].data_ptr(), t["k"].data_ptr(), t["v"].data_ptr(), o.data_ptr(),
                                          lse.data_ptr(), w.B, w.H, w.kv_heads, w.Nq, w.Nk, w.d, None, w.scale,
                                          int(w.causal), dt, 0, ws.data_ptr(), ws.numel(), stream)
            if st != 0:
                raise ea.AttnError(st, "attn_fwd_kvcache_gqa")
    else:
        ws = torch.empty(ea.attn_fwd_kvcache_workspace_bytes(w.B, w.H, w.Nq, w.Nk, w.d, 0), dtype=torch.uint8,
                         device=dev)
        splits = ea.attn_fwd_kvcache_splits(w.B, w.H, w.Nq, w.Nk, w.d, 0)

        def step(i):
            t = sets[i % copies]
            ea.attn_fwd_kvcache(t["q"], t["k"], t["v"], o, lse, w.scale, w.causal, ws)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ms_per_step, prof = timed_passes(lambda i: step(args.warmup + i), args.steps)
    copy_calibration(args.copy_calibration_bytes, dev)
    kernels = {kname: {"launches": n, "avg_ms": round(t / n, 5)} for kname, (n, t) in prof.items() if n}
    # the split kernel reads K, V and Q once: its algorithmic bytes (its
    # workspace writes, 4 (d + 4) bytes per query row and split, are not counted)
    split_bytes = w.kv_bytes() + w.B * w.H * w.Nq * w.d * 2
    avg_ms = prof["kv_split"][1] / prof["kv_split"][0]
    achieved = split_bytes / (avg_ms * 1e-3) / 1e9
    line = {
        "metric": "KV-cache attention forward GB/s (K, V, Q read + O, lse written, per call)",
        "value": round(w.io_bytes() / (ms_per_step * 1e-3) / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "Hkv": w.kv_heads, "Nq": w.Nq, "Nk": w.Nk, "d": w.d,
                   "causal": w.causal, "splits": splits, "input_copies": copies, "seed": w.seed},
        "kernels": kernels,
        "roofline": {
            "kernel": "kv_split",
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic("kv_split", w.name),
        },
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_kv(w, x, min(args.cpu_baseline_seconds, 5.0))
    print(json.dumps(line), flush=True)
    return 0


class ClockSampler:
    """Samples the GPU's current shader clock (sysfs pp_dpm_sclk, the line marked
    '*') every few milliseconds on a host thread while a timed region runs."""

    def __init__(self, period_s: float = 0.005):
        import glob
        import threading
        paths = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        self.path = paths[0] if paths else None
        self.period = period_s
        self.samples = []
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    def _read(self):
        try:
            with open(self.path) as f:
                for line in f:
                    if line.rstrip().endswith("*"):
                        return float(line.split(":")[1].strip().split("Mhz")[0].split("MHz")[0])
        except (OSError, ValueError, IndexError):
            return None
        return None

    def _run(self):
        while not self._stop.is_set():
            v = self._read()
            if v is not None:
                self.samples.append(v)
            self._stop.wait(self.period)

    def __enter__(self):
        if self.path:
            self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self.path:
            self._thread.join()

    def summary(self):
        if not self.samples:
            return None
        v = sorted(self.samples)
        return {"median_mhz": v[len(v) // 2], "min_mhz": v[0], "max_mhz": v[-1], "samples": len(v),
                "source": "sysfs pp_dpm_sclk"}


def time_split(fwd, bwd, est_step_ms: float, min_reps: int = 20, min_span_s: float = 0.5):
    """Forward and backward timed separately: every step bracketed by events
    (fwd between the first two, bwd between the last two), at least min_reps
    steps and min_span_s seconds of GPU time; medians, with the clock sampled
    meanwhile."""
    import math
    import statistics

    import torch

    reps = max(min_reps, int(math.ceil(1.25 * min_span_s * 1e3 / max(est_step_ms, 1e-3))))
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(reps)]
    torch.cuda.synchronize()
    with ClockSampler() as clk:
        for e in ev:
            e[0].record()
            fwd()
            e[1].record()
            if bwd is not None:
                bwd()
            e[2].record()
        torch.cuda.synchronize()
    f = [e[0].elapsed_time(e[1]) for e in ev]
    b = [e[1].elapsed_time(e[2]) for e in ev] if bwd is not None else [0.0] * reps
    steps = [x + y for x, y in zip(f, b)]
    return {"reps": reps, "span_s": round(ev[0][0].elapsed_time(ev[-1][2]) * 1e-3, 3),
            "fwd_ms_median": round(statistics.median(f), 5),
            "bwd_ms_median": round(statistics.median(b), 5) if bwd is not None else None,
            "step_ms_median": round(statistics.median(steps), 5),
            "step_ms_min": round(min(steps), 5), "step_ms_max": round(max(steps), 5),
            "clock": clk.summary()}


def training_setup(w, dev, alibi: bool = False, dropout: float = 0.0, dropout_seed: int = 0):
    """Inputs resident on the device and the forward / backward calls of one
    step through the C ABI (plain, ALiBi or dropout entry points)."""
    import torch
    import exact_attention_66_amd as ea
    import workloads

    x = workloads.make_inputs(w)
    q, k, v = (x[n].to(dev) for n in ("q", "k", "v"))
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    do = x["do"].to(dev) if w.backward else None
    if w.backward:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
        ws = torch.empty(ea.attn_bwd_workspace_bytes(*w.shape()), dtype=torch.uint8, device=dev)
    lib = ea.load()
    stream = torch.cuda.current_stream().cuda_stream or None
    dt = ea.ATTN_DTYPE_BF16 if w.dtype == "bf16" else ea.ATTN_DTYPE_FP16

    def check(st, what):
        if st != 0:
            raise ea.AttnError(st, what)

    if alibi:
        slopes = torch.tensor([2.0 ** (-8.0 * (h + 1) / w.H) for h in range(w.H)], dtype=torch.float32, device=dev)

        def fwd():
            check(lib.attn_fwd_alibi(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), w.B,
                                     w.H, w.N, w.d, slopes.data_ptr(), w.scale, int(w.causal), dt, stream),
                  "attn_fwd_alibi")

        def bwd():
            check(lib.attn_bwd_alibi(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                                     lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), w.B, w.H, w.N,
                                     w.d, slopes.data_ptr(), w.scale, int(w.causal), dt, ws.data_ptr(), ws.numel(),
                                     stream), "attn_bwd_alibi")
    elif dropout > 0:
        def fwd():
            check(lib.attn_fwd_dropout(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), w.B,
                                       w.H, w.N, w.d, w.scale, int(w.causal), dt, dropout, dropout_seed, 0, stream),
                  "attn_fwd_dropout")

        def bwd():
            check(lib.attn_bwd_dropout(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                                       lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), w.B, w.H, w.N,
                                       w.d, w.scale, int(w.causal), dt, dropout, dropout_seed, 0, ws.data_ptr(),
                                       ws.numel(), stream), "attn_bwd_dropout")
    else:
        def fwd():
            check(lib.attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), w.B, w.H,
                               w.N, w.d, w.scale, int(w.causal), dt, stream), "attn_fwd")

        def bwd():
            check(lib.attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                               lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), w.B, w.H, w.N, w.d,
                               w.scale, int(w.causal), dt, ws.data_ptr(), ws.numel(), stream), "attn_bwd")
    return x, fwd, (bwd if w.backward else None)


def kernel_summary(w, prof, traffic_key, with_traffic: bool = True):
    """Per-kernel average durations and the roofline of the dominant kernel:
    the counted flops each kernel carries (the backward's five products are
    S, dP, dV, dK in bwd_dkdv and dQ in bwd_dq, which also recomputes S and
    dP: extra work that is not counted) over its average launch duration."""
    flops_per_launch = {"fwd": w.fwd_flops(), "bwd_dkdv": 0.8 * w.bwd_flops(), "bwd_dq": 0.2 * w.bwd_flops()}
    kernels = {kname: {"launches": n, "avg_ms": round(t / n, 5)} for kname, (n, t) in prof.items() if n}
    dominant = max((kname for kname in kernels if kname in flops_per_launch), key=lambda kname: prof[kname][1])
    avg_ms = prof[dominant][1] / prof[dominant][0]
    achieved = flops_per_launch[dominant] / (avg_ms * 1e-3) / 1e12
    roofline = {
        "kernel": dominant,
        "bound": "mfma",
        "achieved": round(achieved, 2),
        "peak": PEAK_TFLOPS,
        "unit": "TFLOP/s",
        "frac": round(achieved / PEAK_TFLOPS, 4),
        "traffic": measured_traffic(dominant, traffic_key) if with_traffic else None,
    }
    return kernels, roofline


def split_summary(w, split):
    """TFLOP/s from the split medians: fwd+bwd counted flops over the sum of
    the forward and backward medians, and each pass on its own; % of the
    published peak and of the peak at the sampled clock."""
    fwd_ms, bwd_ms = split["fwd_ms_median"], split["bwd_ms_median"] or 0.0
    tot = w.fwd_flops() + w.bwd_flops()
    out = {"tflops": round(tot / ((fwd_ms + bwd_ms) * 1e-3) / 1e12, 2),
           "fwd_tflops": round(w.fwd_flops() / (fwd_ms * 1e-3) / 1e12, 2)}
    if w.backward:
        out["bwd_tflops"] = round(w.bwd_flops() / (bwd_ms * 1e-3) / 1e12, 2)
    out["pct_of_peak"] = round(100 * out["tflops"] / PEAK_TFLOPS, 2)
    clk = split.get("clock")
    if clk:
        peak_at_clock = PEAK_TFLOPS * clk["median_mhz"] / PEAK_CLOCK_MHZ
        out["pct_of_peak_at_clock"] = round(100 * out["tflops"] / peak_at_clock, 2)
    return out


def bench_other_workload(w, dev, warmup: int):
    """One more training workload, as its own summary (not the line's value)."""
    import torch
    import exact_attention_66_amd as ea

    x, fwd, bwd = training_setup(w, dev)
    del x
    for _ in range(max(warmup, 2)):
        fwd()
        if bwd is not None:
            bwd()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        fwd()
        if bwd is not None:
            bwd()
    e1.record()
    torch.cuda.synchronize()
    split = time_split(fwd, bwd, e0.elapsed_time(e1) / 5)
    ea.attn_profile_start()
    for _ in range(10):
        fwd()
        if bwd is not None:
            bwd()
    torch.cuda.synchronize()
    kernels, roofline = kernel_summary(w, ea.attn_profile_stop(), w.name)
    out = {"config": {"B": w.B, "H": w.H, "N": w.N, "d": w.d, "dtype": w.dtype, "causal": w.causal,
                      "passes": "fwd+bwd" if w.backward else "fwd", "seed": w.seed}}
    out.update(split_summary(w, split))
    out["timing"] = split
    out["kernels"] = kernels
    out["roofline"] = roofline
    return out


def main() -> int:
    import workloads

    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=workloads.HEADLINE,
                    choices=sorted(workloads.WORKLOADS) + sorted(workloads.KV_WORKLOADS))
    ap.add_argument("--cpu-baseline-seconds", type=float, default=20.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="measure only --workload (by default the headline run also measures every other "
                         "training workload)")
    ap.add_argument("--copy-calibration-bytes", type=int, default=0,
                    help="after the timed steps, also run a plain device copy of this many bytes "
                         "(reference kernel for scaling the HBM byte counters)")
    ap.add_argument("--alibi", action="store_true",
                    help="run the ALiBi entry points (slopes 2^(-8(h+1)/H)) on the same workload")
    ap.add_argument("--dropout", type=float, default=0.0, metavar="P",
                    help="run the dropout entry points with probability P (seed --dropout-seed) on the same workload")
    ap.add_argument("--dropout-seed", type=int, default=2026)
    ap.add_argument("--record-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU run: turn rocprofv3 FETCH_SIZE / WRITE_SIZE counter files into the "
                         "workload's HBM bytes per launch in profiles/hbm_traffic.json")
    args = ap.parse_args()

    # counter records of the dropout instantiations are kept apart from the plain ones
    traffic_key = args.workload + ("+dropout" if args.dropout > 0 else "")
    if args.record_traffic:
        return record_traffic(*args.record_traffic, traffic_key)

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

    if args.workload in workloads.KV_WORKLOADS:
        return bench_kvcache(args, workloads.KV_WORKLOADS[args.workload])

    w = workloads.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    x, fwd, bwd = training_setup(w, dev, args.alibi, args.dropout, args.dropout_seed)

    def step(i=0):
        fwd()
        if bwd is not None:
            bwd()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ms_per_step, prof = timed_passes(step, args.steps)
    split = time_split(fwd, bwd, ms_per_step)

    copy_calibration(args.copy_calibration_bytes, dev)

    flops = w.fwd_flops() + w.bwd_flops()
    value = flops / (ms_per_step * 1e-3) / 1e12
    kernels, roofline = kernel_summary(w, prof, traffic_key, with_traffic=not args.alibi)
    timing = dict(split_summary(w, split), **split)

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
                   "passes": "fwd+bwd" if w.backward else "fwd", "seed": w.seed, "alibi": bool(args.alibi),
                   "dropout_p": args.dropout},
        "pct_of_peak": round(100 * value / PEAK_TFLOPS, 2),
        "timing": timing,
        "kernels": kernels,
        "roofline": roofline,
    }
    if not (args.no_other_workloads or args.alibi or args.dropout > 0 or args.workload != workloads.HEADLINE):
        others = {}
        for name, wo in workloads.WORKLOADS.items():
            if name == w.name:
                continue
            others[name] = bench_other_workload(wo, dev, args.warmup)
            torch.cuda.empty_cache()
        line["workloads"] = others
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, x, args.cpu_baseline_seconds,
                                            (args.dropout, args.dropout_seed, 0) if args.dropout > 0 else None)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
