"""Capture of the C-ABI calls into a HIP graph (GPU).

Every entry point only enqueues kernels on the caller's stream (no
allocation, no memset, no synchronisation), so a graph captured around a
forward, a backward and a KV-cache call replays them.  Each replay, with
eager work and synchronisations between replays, must give bitwise the
outputs of the eager calls (the kernels are deterministic).
"""
import pytest
import torch

import workloads
from parity import log, require_gpu

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager():
    ea = require_gpu()
    w = workloads.Workload("graph", 2, 4, 320, 128, "bf16", True, True, seed=61001)
    x = workloads.make_inputs(w)
    q, k, v, do = (x[n].cuda() for n in ("q", "k", "v", "do"))
    kw = workloads.KvWorkload("graph_kv", 2, 4, 3, 1500, 128, "bf16", True, seed=61002)
    xk = workloads.make_kv_inputs(kw)
    qk, kk, vk = (xk[n].cuda() for n in ("q", "k", "v"))

    # every buffer the calls touch exists before capture
    o, lse = torch.empty_like(q), torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(ea.attn_bwd_workspace_bytes(w.B, w.H, w.N, w.d), dtype=torch.uint8, device="cuda")
    ok, lk = torch.empty_like(qk), torch.empty((kw.B, kw.H, kw.Nq), dtype=torch.float32, device="cuda")
    wsk = torch.empty(ea.attn_fwd_kvcache_workspace_bytes(kw.B, kw.H, kw.Nq, kw.Nk, kw.d), dtype=torch.uint8,
                      device="cuda")

    def calls():
        ea.attn_fwd(q, k, v, o, lse, w.scale, True)
        ea.attn_bwd(q, k, v, o, do, lse, dq, dk, dv, w.scale, True, ws)
        ea.attn_fwd_kvcache(qk, kk, vk, ok, lk, kw.scale, True, wsk)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()                      # eager run on the capture stream first
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    eager = [t.clone() for t in (o, lse, dq, dk, dv, ok, lk)]

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in (o, dq, dk, dv, ok):
            t.fill_(float("nan"))    # eager work between replays
        lse.fill_(0.0)
        lk.fill_(0.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, t, e in zip(("O", "lse", "dQ", "dK", "dV", "O_kv", "lse_kv"), (o, lse, dq, dk, dv, ok, lk), eager):
            assert torch.equal(t, e), f"replay {rep}: {name} differs from the eager result"
        log(f"graph replay {rep}: all outputs bitwise equal to eager")
