"""Forward parity of the HIP kernels against the fp64 oracle (runs on the GPU).

Small shapes are compared element by element over every head; they span
several query blocks and key tiles and a ragged last query block.  The full
workload sizes are compared over every element in test_gpu_fullsize.py.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import check_lse, check_o, f64, log, require_gpu

pytestmark = pytest.mark.gpu


def _run_fwd(ea, inputs, scale, causal):
    q, k, v = (inputs[n].cuda() for n in ("q", "k", "v"))
    o, lse = ea.forward(q, k, v, scale=scale, causal=causal)
    torch.cuda.synchronize()
    return o, lse


SMALL = [
    # (B, H, N, d, dtype, causal)
    (1, 2, 64, 64, "bf16", False),
    (1, 2, 64, 128, "bf16", True),
    (2, 3, 192, 64, "bf16", True),
    (1, 2, 320, 128, "bf16", True),      # N not a multiple of the 128-query block
    (1, 2, 320, 64, "fp16", False),
    (2, 2, 512, 128, "fp16", True),
    (1, 1, 1024, 128, "bf16", False),
    (1, 2, 1088, 64, "fp16", True),
]


@pytest.mark.parametrize("B,H,N,d,dt,causal", SMALL)
def test_forward_small_all_elements(B, H, N, d, dt, causal):
    ea = require_gpu()
    w = workloads.Workload("small", B, H, N, d, dt, causal, False, seed=7000 + N + d + B * 10 + H)
    log(f"forward small {w}")
    x = workloads.make_inputs(w)
    o, lse = _run_fwd(ea, x, w.scale, causal)
    o_ref, lse_ref = oracle.forward(workloads.to_f64_numpy(x["q"]), workloads.to_f64_numpy(x["k"]),
                                    workloads.to_f64_numpy(x["v"]), w.scale, causal)
    check_o(f64(o), o_ref, dt)
    check_lse(f64(lse), lse_ref)


def test_forward_small_workload_exact_size():
    """The small forward-only workload (B=1, H=4, N=256, d=64, non-causal) at its full size."""
    ea = require_gpu()
    w = workloads.WORKLOADS["fwd_b1h4n256d64"]
    log(f"forward {w.name}")
    x = workloads.make_inputs(w)
    o, lse = _run_fwd(ea, x, w.scale, w.causal)
    o_ref, lse_ref = oracle.forward(*(workloads.to_f64_numpy(x[n]) for n in ("q", "k", "v")), w.scale, w.causal)
    check_o(f64(o), o_ref, w.dtype)
    check_lse(f64(lse), lse_ref)


@pytest.mark.parametrize("dt", ["bf16", "fp16"])
@pytest.mark.parametrize("causal", [False, True])
def test_forward_special_inputs(dt, causal):
    """Uniform scores (Q = 0), strongly peaked rows (the running max jumps
    many times, exercising the rescale path), and constant V."""
    ea = require_gpu()
    B, H, N, d = 1, 2, 384, 128
    w = workloads.Workload("special", B, H, N, d, dt, causal, False, seed=8100)
    x = workloads.make_inputs(w)
    cases = {}
    cases["q_zero"] = dict(x, q=torch.zeros_like(x["q"]))
    # keys growing along the sequence: each new tile raises the row max
    ramp = torch.linspace(0.5, 6.0, N).view(1, 1, N, 1)
    cases["ramp"] = dict(x, q=(torch.ones(B, H, N, d) * 0.25).to(w.torch_dtype),
                         k=(ramp * torch.ones(B, H, N, d) / 4).to(w.torch_dtype))
    cases["peaky_x8"] = dict(x, q=(x["q"].float() * 4).to(w.torch_dtype), k=(x["k"].float() * 2).to(w.torch_dtype))
    cases["v_const"] = dict(x, v=torch.full_like(x["v"], 1.5))
    for cname, xc in cases.items():
        log(f"forward special {cname} {dt} causal={causal}")
        o, lse = _run_fwd(ea, xc, w.scale, causal)
        o_ref, lse_ref = oracle.forward(*(workloads.to_f64_numpy(xc[n]) for n in ("q", "k", "v")), w.scale, causal)
        check_o(f64(o), o_ref, dt, what=f"O {cname}")
        check_lse(f64(lse), lse_ref, what=f"lse {cname}")


def test_forward_deterministic():
    ea = require_gpu()
    w = workloads.Workload("det", 2, 4, 1024, 128, "bf16", True, False, seed=8200)
    x = workloads.make_inputs(w)
    o1, l1 = _run_fwd(ea, x, w.scale, True)
    o2, l2 = _run_fwd(ea, x, w.scale, True)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_forward_writes_every_output_element():
    """Outputs start as NaN; every element must be overwritten."""
    ea = require_gpu()
    w = workloads.Workload("nan", 1, 3, 448, 64, "fp16", True, False, seed=8300)
    x = workloads.make_inputs(w)
    q, k, v = (x[n].cuda() for n in ("q", "k", "v"))
    o = torch.full_like(q, float("nan"))
    lse = torch.full((1, 3, 448), float("nan"), device="cuda")
    ea.attn_fwd(q, k, v, o, lse, w.scale, True)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all().item() and torch.isfinite(lse).all().item()


def test_forward_on_side_stream():
    ea = require_gpu()
    w = workloads.Workload("stream", 1, 2, 256, 64, "bf16", False, False, seed=8400)
    x = workloads.make_inputs(w)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        q, k, v = (x[n].cuda() for n in ("q", "k", "v"))
        o, lse = ea.forward(q, k, v, scale=w.scale, causal=False)
    s.synchronize()
    o_ref, lse_ref = oracle.forward(*(workloads.to_f64_numpy(x[n]) for n in ("q", "k", "v")), w.scale, False)
    check_o(f64(o), o_ref, "bf16")
    check_lse(f64(lse), lse_ref)
