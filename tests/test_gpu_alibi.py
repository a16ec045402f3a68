"""Parity of the ALiBi entry points (linear position bias) with the fp64 oracle (GPU).

The bias -m_h |p_i - j| is added to the scaled scores before the softmax
(p_i the query's position).  Slopes follow the usual geometric choice
m_h = 2^(-8 (h + 1) / H); the oracle takes the same fp32 values.  Every
element is compared on small and ragged shapes; the headline-sized
training shape is checked on sampled heads.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import check_grad, check_lse, check_o, f64, log, require_gpu

pytestmark = pytest.mark.gpu


def _slopes(H):
    return torch.tensor([2.0 ** (-8.0 * (h + 1) / H) for h in range(H)], dtype=torch.float32)


def _np(t):
    return workloads.to_f64_numpy(t)


CASES = [(1, 4, 256, 64, "bf16", True), (2, 2, 333, 128, "bf16", False), (1, 8, 200, 128, "fp16", True),
         (2, 3, 1000, 64, "bf16", True), (1, 2, 64, 128, "fp16", False)]


@pytest.mark.parametrize("B,H,N,d,dt,causal", CASES)
def test_alibi_forward_backward_all_elements(B, H, N, d, dt, causal):
    ea = require_gpu()
    w = workloads.Workload("alibi", B, H, N, d, dt, causal, True, seed=51000 + N + d + H)
    x = workloads.make_inputs(w)
    sl = _slopes(H)
    q, k, v, do = (x[n].cuda() for n in ("q", "k", "v", "do"))
    log(f"alibi fwd+bwd B={B} H={H} N={N} d={d} {dt} causal={causal}")
    o, lse = ea.forward_alibi(q, k, v, sl, scale=w.scale, causal=causal)
    dq, dk, dv = ea.backward_alibi(q, k, v, o, lse, do, sl, scale=w.scale, causal=causal)
    torch.cuda.synchronize()
    args = [_np(x[n]) for n in ("q", "k", "v")]
    o_ref, lse_ref = oracle.forward(*args, w.scale, causal, alibi_slopes=sl.double().numpy())
    check_o(f64(o), o_ref, dt)
    check_lse(f64(lse), lse_ref)
    grads = oracle.backward(*args, _np(x["do"]), w.scale, causal, alibi_slopes=sl.double().numpy())
    for name, g, gr in zip(("dQ", "dK", "dV"), (dq, dk, dv), grads):
        check_grad(f64(g), gr, name)


@pytest.mark.parametrize("Nq,Nk,splits", [(1, 4096, 0), (8, 1111, 0), (40, 300, 5)])
def test_alibi_kvcache(Nq, Nk, splits):
    ea = require_gpu()
    w = workloads.KvWorkload("alibi_kv", 2, 4, Nq, Nk, 128, "bf16", True, seed=52000 + Nk)
    x = workloads.make_kv_inputs(w)
    sl = _slopes(w.H)
    q, k, v = (x[n].cuda() for n in ("q", "k", "v"))
    log(f"alibi kvcache Nq={Nq} Nk={Nk} splits={splits}")
    o, lse = ea.forward_kvcache_alibi(q, k, v, sl, scale=w.scale, causal=True, num_splits=splits)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.forward(*(_np(x[n]) for n in ("q", "k", "v")), w.scale, True,
                                    alibi_slopes=sl.double().numpy())
    check_o(f64(o), o_ref, "bf16")
    check_lse(f64(lse), lse_ref)


def test_alibi_headline_shape_sampled_heads():
    """B=4, H=32, N=4096, d=128 causal bf16 with ALiBi: two whole heads against the oracle."""
    ea = require_gpu()
    w = workloads.WORKLOADS["causal_b4h32n4096d128"]
    x = workloads.make_inputs(w)
    sl = _slopes(w.H)
    q, k, v, do = (x[n].cuda() for n in ("q", "k", "v", "do"))
    log("alibi headline shape B=4 H=32 N=4096 d=128")
    o, lse = ea.forward_alibi(q, k, v, sl, scale=w.scale, causal=True)
    dq, dk, dv = ea.backward_alibi(q, k, v, o, lse, do, sl, scale=w.scale, causal=True)
    torch.cuda.synchronize()
    for b, h in ((0, 0), (3, 31)):
        args = [_np(x[n][b, h]) for n in ("q", "k", "v")]
        m = float(sl[h])
        o_ref, lse_ref = oracle.forward_head(*args, w.scale, True, alibi_slope=m)
        check_o(f64(o[b, h]), o_ref, "bf16")
        check_lse(f64(lse[b, h]), lse_ref)
        grads = oracle.backward_head(*args, _np(x["do"][b, h]), w.scale, True, alibi_slope=m)
        for name, g, gr in zip(("dQ", "dK", "dV"), (dq[b, h], dk[b, h], dv[b, h]), grads):
            check_grad(f64(g), gr, f"{name}[{b},{h}]")
