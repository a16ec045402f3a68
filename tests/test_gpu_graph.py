"""Capture of the C-ABI calls into a HIP graph (GPU).

Every entry point only enqueues kernels on the caller's stream (no
allocation, no memset, no synchronisation), so a graph captured around a
forward, a backward, a KV-cache call and a forward and backward with dropout
replays them.  Each replay, with
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
    od, lsed = torch.empty_like(q), torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda")
    dqd, dkd, dvd = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    lib = ea.load()
    dt = ea.ATTN_DTYPE_BF16

    def calls():
        ea.attn_fwd(q, k, v, o, lse, w.scale, True)
        ea.attn_bwd(q, k, v, o, do, lse, dq, dk, dv, w.scale, True, ws)
        ea.attn_fwd_kvcache(qk, kk, vk, ok, lk, kw.scale, True, wsk)
        st = torch.cuda.current_stream().cuda_stream or None
        assert lib.attn_fwd_dropout(q.data_ptr(), k.data_ptr(), v.data_ptr(), od.data_ptr(), lsed.data_ptr(), w.B,
                                    w.H, w.N, w.d, w.scale, 1, dt, 0.2, 99, 4, st) == 0
        assert lib.attn_bwd_dropout(q.data_ptr(), k.data_ptr(), v.data_ptr(), od.data_ptr(), do.data_ptr(),
                                    lsed.data_ptr(), dqd.data_ptr(), dkd.data_ptr(), dvd.data_ptr(), w.B, w.H, w.N,
                                    w.d, w.scale, 1, dt, 0.2, 99, 4, ws.data_ptr(), ws.numel(), st) == 0

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()                      # eager run on the capture stream first
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    eager = [t.clone() for t in (o, lse, dq, dk, dv, ok, lk, od, lsed, dqd, dkd, dvd)]

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in (o, dq, dk, dv, ok, od, dqd, dkd, dvd):
            t.fill_(float("nan"))    # eager work between replays
        lse.fill_(0.0)
        lk.fill_(0.0)
        lsed.fill_(0.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        names = ("O", "lse", "dQ", "dK", "dV", "O_kv", "lse_kv", "O_drop", "lse_drop", "dQ_drop", "dK_drop", "dV_drop")
        outs = (o, lse, dq, dk, dv, ok, lk, od, lsed, dqd, dkd, dvd)
        for name, t, e in zip(names, outs, eager):
            assert torch.equal(t, e), f"replay {rep}: {name} differs from the eager result"
        log(f"graph replay {rep}: all outputs bitwise equal to eager")
