"""Backward parity of the HIP kernels against the fp64 oracle (runs on the GPU).

The GPU forward output (O, lse) feeds the GPU backward exactly as in
training; the oracle computes its gradients from the same rounded inputs.
Small shapes are compared over every head; the full workload sizes are
compared over every element, with the gradient invariants on every head, in
test_gpu_fullsize.py.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import check_grad, f64, log, require_gpu

pytestmark = pytest.mark.gpu


def _run(ea, x, scale, causal):
    q, k, v, do = (x[n].cuda() for n in ("q", "k", "v", "do"))
    o, lse = ea.forward(q, k, v, scale=scale, causal=causal)
    dq, dk, dv = ea.backward(q, k, v, o, lse, do, scale=scale, causal=causal)
    torch.cuda.synchronize()
    return (q, k, v, do, o, lse), (dq, dk, dv)


SMALL = [
    (1, 2, 64, 64, "bf16", False),
    (1, 2, 64, 128, "bf16", True),
    (2, 3, 192, 64, "bf16", True),       # key blocks of 128 with a ragged last block
    (1, 2, 320, 128, "bf16", True),
    (1, 2, 320, 64, "fp16", False),
    (2, 2, 512, 128, "fp16", True),
    (1, 1, 1024, 128, "bf16", False),
    (1, 2, 1088, 64, "fp16", True),
    (3, 48, 256, 128, "bf16", True),     # more dK/dV units than resident workgroups:
    (4, 72, 256, 64, "fp16", True),      # workgroups run several units in turn
]


@pytest.mark.parametrize("B,H,N,d,dt,causal", SMALL)
def test_backward_small_all_elements(B, H, N, d, dt, causal):
    ea = require_gpu()
    w = workloads.Workload("small", B, H, N, d, dt, causal, True, seed=9000 + N + d + 10 * B + H)
    log(f"backward small {w}")
    x = workloads.make_inputs(w)
    _, grads = _run(ea, x, w.scale, causal)
    ref = oracle.backward(*(workloads.to_f64_numpy(x[n]) for n in ("q", "k", "v", "do")), w.scale, causal)
    for name, g, gr in zip(("dQ", "dK", "dV"), grads, ref):
        check_grad(f64(g), gr, name)


def test_backward_deterministic():
    """No atomics: every gradient element is accumulated by one lane, so runs are bitwise equal."""
    ea = require_gpu()
    w = workloads.Workload("det", 2, 4, 1024, 128, "bf16", True, True, seed=9100)
    x = workloads.make_inputs(w)
    _, (dq1, dk1, dv1) = _run(ea, x, w.scale, True)
    _, (dq2, dk2, dv2) = _run(ea, x, w.scale, True)
    assert torch.equal(dk1, dk2) and torch.equal(dv1, dv2) and torch.equal(dq1, dq2)


def test_backward_writes_every_output_element():
    ea = require_gpu()
    w = workloads.Workload("nan", 1, 3, 448, 64, "fp16", True, True, seed=9200)
    x = workloads.make_inputs(w)
    q, k, v, do = (x[n].cuda() for n in ("q", "k", "v", "do"))
    o, lse = ea.forward(q, k, v, scale=w.scale, causal=True)
    dq, dk, dv = (torch.full_like(q, float("nan")) for _ in range(3))
    ws = torch.full((ea.attn_bwd_workspace_bytes(1, 3, 448, 64),), 255, dtype=torch.uint8, device="cuda")
    ea.attn_bwd(q, k, v, o, do, lse, dq, dk, dv, w.scale, True, ws)
    torch.cuda.synchronize()
    assert torch.isfinite(dq).all().item() and torch.isfinite(dk).all().item() and torch.isfinite(dv).all().item()


@pytest.mark.parametrize("causal", [False, True])
def test_backward_special_inputs(causal):
    """Identical keys give dQ = 0; identical values give dQ = dK = 0; a
    peaky (x4 / x2) input exercises large lse values."""
    ea = require_gpu()
    B, H, N, d = 1, 2, 256, 128
    w = workloads.Workload("special", B, H, N, d, "bf16", causal, True, seed=9300)
    x = workloads.make_inputs(w)
    same_k = dict(x, k=x["k"][:, :, :1].expand(-1, -1, N, -1).contiguous())
    _, (dq, dk, dv) = _run(ea, same_k, w.scale, causal)
    assert dq.float().abs().max().item() <= 1e-2 * (1 + dk.float().abs().max().item())
    same_v = dict(x, v=x["v"][:, :, :1].expand(-1, -1, N, -1).contiguous())
    _, (dq, dk, dv) = _run(ea, same_v, w.scale, causal)
    assert dq.float().abs().max().item() <= 1e-2 and dk.float().abs().max().item() <= 1e-2
    peaky = dict(x, q=(x["q"].float() * 4).to(torch.bfloat16), k=(x["k"].float() * 2).to(torch.bfloat16))
    _, grads = _run(ea, peaky, w.scale, causal)
    ref = oracle.backward(*(workloads.to_f64_numpy(peaky[n]) for n in ("q", "k", "v", "do")), w.scale, causal)
    for name, g, gr in zip(("dQ", "dK", "dV"), grads, ref):
        check_grad(f64(g), gr, f"peaky {name}")


def test_backward_workspace_reuse_and_side_stream():
    ea = require_gpu()
    w = workloads.Workload("ws", 1, 2, 512, 64, "bf16", True, True, seed=9400)
    x = workloads.make_inputs(w)
    ws = torch.empty(ea.attn_bwd_workspace_bytes(1, 2, 512, 64), dtype=torch.uint8, device="cuda")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        q, k, v, do = (x[n].cuda() for n in ("q", "k", "v", "do"))
        o, lse = ea.forward(q, k, v, scale=w.scale, causal=True)
        g1 = ea.backward(q, k, v, o, lse, do, scale=w.scale, causal=True, workspace=ws)
        g2 = ea.backward(q, k, v, o, lse, do, scale=w.scale, causal=True, workspace=ws)
    s.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(g1, g2))
    ref = oracle.backward(*(workloads.to_f64_numpy(x[n]) for n in ("q", "k", "v", "do")), w.scale, True)
    for name, g, gr in zip(("dQ", "dK", "dV"), g2, ref):
        check_grad(f64(g), gr, name)
