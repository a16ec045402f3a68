"""Parity of the ALiBi entry points (linear position bias) with the fp64 oracle (GPU).

The bias -m_h |p_i - j| is added to the scaled scores before the softmax
(p_i the query's position).  Slopes follow the usual geometric choice
m_h = 2^(-8 (h + 1) / H); the oracle takes the same fp32 values.  Every
element is compared on small and ragged shapes and on the headline-sized
training shape (through the per-head oracle pool).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from oracle_pool import compare_full
from parity import GRAD_REL_FRO, LSE_MAX, O_MEAN, check_grad, check_lse, check_o, f64, log, require_gpu

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


@pytest.mark.timeout(900)
def test_alibi_headline_shape_every_element():
    """B=4, H=32, N=4096, d=128 causal bf16 with ALiBi: every element of O, lse, dQ, dK and dV
    against the oracle, with the bounds of the full-size parity tests."""
    ea = require_gpu()
    w = workloads.WORKLOADS["causal_b4h32n4096d128"]
    x = workloads.make_inputs(w)
    sl = _slopes(w.H)
    q, k, v, do = (x[n].cuda() for n in ("q", "k", "v", "do"))
    log("alibi headline shape B=4 H=32 N=4096 d=128, every element")
    o, lse = ea.forward_alibi(q, k, v, sl, scale=w.scale, causal=True)
    dq, dk, dv = ea.backward_alibi(q, k, v, o, lse, do, sl, scale=w.scale, causal=True)
    torch.cuda.synchronize()
    m = compare_full(w, x, o.cpu(), lse.cpu(), tuple(g.cpu() for g in (dq, dk, dv)),
                     alibi_slopes=sl.double().numpy())
    log(f"  O over {m['o_elements']} elements: max|err| {m['o_max']:.3e} mean|err| {m['o_mean']:.3e}; "
        f"lse max|err| {m['lse_max']:.3e}; rel. Frobenius dq {m['dq_rel_fro']:.3e} dk {m['dk_rel_fro']:.3e} "
        f"dv {m['dv_rel_fro']:.3e}")
    assert m["finite"] and all(m[g + "_finite"] for g in ("dq", "dk", "dv"))
    assert m["o_over"] == 0, m.get("o_worst_over")
    assert m["o_mean"] <= O_MEAN
    assert m["lse_max"] <= LSE_MAX
    for g in ("dq", "dk", "dv"):
        assert m[g + "_rel_fro"] <= GRAD_REL_FRO, (g, m[g + "_rel_fro"])
