"""Parity at sequence lengths that are not a multiple of the tile sizes (runs on the GPU).

Any N >= 1 is accepted.  The last query block and the last key tile then
run past the end of the sequence: the forward clamps its copies of that tile
to the last key and masks the keys past the end; the backward pads its
workspace to a multiple of 64 tokens (padded queries get P = 0) and takes
the last partial 64-token tile of Q, dO, K, V from zero-padded copies.  These
tests compare every element with the fp64 oracle, check that nothing past
row N - 1 of an output is written, and include rows whose every score is
very negative, where an unmasked padded key would overflow exp().
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import check_grad, check_lse, check_o, f64, log, require_gpu

pytestmark = pytest.mark.gpu

CASES = [
    # (B, H, N, d, dtype, causal): N below, at and across tile edges (32-key
    # blocks, 64-token tiles, 128-key forward tiles, 128-key dK/dV units,
    # 256-query blocks)
    (1, 2, 1, 64, "bf16", False),
    (1, 2, 1, 128, "fp16", True),
    (2, 1, 7, 128, "bf16", True),
    (1, 3, 33, 64, "fp16", False),
    (1, 2, 65, 128, "bf16", False),
    (2, 2, 100, 64, "bf16", True),
    (1, 2, 127, 128, "fp16", True),
    (1, 2, 129, 64, "bf16", False),
    (1, 2, 200, 128, "bf16", False),
    (1, 2, 255, 64, "fp16", True),
    (1, 2, 257, 128, "bf16", True),
    (1, 1, 321, 128, "fp16", False),
    (2, 2, 1000, 64, "bf16", True),
    (1, 2, 1000, 128, "bf16", False),
]


def _ids(c):
    B, H, N, d, dt, causal = c
    return f"B{B}H{H}N{N}d{d}{dt}{'causal' if causal else ''}"


def _guarded(n, tail, guard, dtype):
    """A [1, 1, n, *tail] array at the start of a [1, 1, n + guard, *tail]
    buffer filled with NaN: (buffer, array).  With B = H = 1 the first n rows
    are contiguous, so the array is a valid kernel argument, and the guard
    rows behind it show any store past row n - 1."""
    big = torch.full((1, 1, n + guard, *tail), float("nan"), dtype=dtype, device="cuda")
    return big, big[:, :, :n]


@pytest.mark.parametrize("B,H,N,d,dt,causal", CASES, ids=[_ids(c) for c in CASES])
def test_ragged_forward_backward_all_elements(B, H, N, d, dt, causal):
    ea = require_gpu()
    w = workloads.Workload("ragged", B, H, N, d, dt, causal, True, seed=11000 + 7 * N + d + B + H)
    log(f"ragged {w}")
    x = workloads.make_inputs(w)
    q, k, v, do = (x[n].cuda() for n in ("q", "k", "v", "do"))
    o, lse = ea.forward(q, k, v, scale=w.scale, causal=causal)
    dq, dk, dv = ea.backward(q, k, v, o, lse, do, scale=w.scale, causal=causal)
    torch.cuda.synchronize()
    xs = [workloads.to_f64_numpy(x[n]) for n in ("q", "k", "v", "do")]
    o_ref, lse_ref = oracle.forward(*xs[:3], w.scale, causal)
    check_o(f64(o), o_ref, dt)
    check_lse(f64(lse), lse_ref)
    ref = oracle.backward(*xs, w.scale, causal)
    for name, g, gr in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref):
        check_grad(f64(g), gr, name)


@pytest.mark.parametrize("N,d,causal", [(100, 64, False), (100, 128, True), (1000, 128, False), (33, 64, True),
                                        (64, 64, False), (64, 128, True), (192, 64, True), (320, 128, False)])
def test_ragged_writes_nothing_past_the_end(N, d, causal):
    """Outputs sit at the start of NaN-filled buffers with 64 guard rows
    behind them: every element of the outputs is written and no guard row is.
    Includes multiples of 64 that are not multiples of 128, where the last
    128-key unit of the dK, dV pass has whole waves past the end."""
    ea = require_gpu()
    w = workloads.Workload("guard", 1, 1, N, d, "bf16", causal, True, seed=11500 + N + d)
    x = workloads.make_inputs(w)
    q, k, v, do = (x[n].cuda() for n in ("q", "k", "v", "do"))
    G = 64
    ob, o = _guarded(N, (d,), G, torch.bfloat16)
    lb, lse = _guarded(N, (), G, torch.float32)
    assert o.is_contiguous() and lse.is_contiguous()
    ea.attn_fwd(q, k, v, o, lse, w.scale, causal)
    grads = [_guarded(N, (d,), G, torch.bfloat16) for _ in range(3)]
    ws = torch.full((ea.attn_bwd_workspace_bytes(1, 1, N, d),), 255, dtype=torch.uint8, device="cuda")
    ea.attn_bwd(q, k, v, o, do, lse, grads[0][1], grads[1][1], grads[2][1], w.scale, causal, ws)
    torch.cuda.synchronize()
    assert torch.isnan(ob[:, :, N:]).all().item() and torch.isnan(lb[:, :, N:]).all().item()
    assert torch.isfinite(o).all().item() and torch.isfinite(lse).all().item()
    for big, view in grads:
        assert torch.isnan(big[:, :, N:]).all().item()
        assert torch.isfinite(view).all().item()
    xs = [workloads.to_f64_numpy(x[n]) for n in ("q", "k", "v", "do")]
    o_ref, lse_ref = oracle.forward(*xs[:3], w.scale, causal)
    check_o(f64(o), o_ref, "bf16")
    check_lse(f64(lse), lse_ref)
    for name, (_, g), gr in zip(("dQ", "dK", "dV"), grads, oracle.backward(*xs, w.scale, causal)):
        check_grad(f64(g), gr, name)


@pytest.mark.parametrize("N,d,causal", [(100, 64, False), (333, 128, False), (200, 128, True)])
def test_ragged_very_negative_scores(N, d, causal):
    """Every score near -100: dimension 0 of every key is c = 4 and of every
    query -A with A c scale = 100, the other dimensions are the usual random
    values.  lse is then near -100 as well, so a padded key that were not
    masked (a zero K row scores 0) would get P = exp(0 - lse) = e^100 and
    poison dQ with inf * 0; and the backward's exponent, taken relative to
    lse, must stay exact at this magnitude."""
    ea = require_gpu()
    w = workloads.Workload("neg", 1, 2, N, d, "bf16", causal, True, seed=11700 + N)
    x = workloads.make_inputs(w)
    c = 4.0
    a = 100.0 / (c * w.scale)
    k = x["k"].float().clone()
    k[..., 0] = c
    q = x["q"].float().clone()
    q[..., 0] = -a
    xc = dict(x, q=q.to(torch.bfloat16), k=k.to(torch.bfloat16))
    qd, kd, vd, dod = (xc[n].cuda() for n in ("q", "k", "v", "do"))
    o, lse = ea.forward(qd, kd, vd, scale=w.scale, causal=causal)
    dq, dk, dv = ea.backward(qd, kd, vd, o, lse, dod, scale=w.scale, causal=causal)
    torch.cuda.synchronize()
    xs = [workloads.to_f64_numpy(xc[n]) for n in ("q", "k", "v", "do")]
    o_ref, lse_ref = oracle.forward(*xs[:3], w.scale, causal)
    assert float(lse_ref.max()) < -80.0, "inputs must make every row's lse very negative"
    check_o(f64(o), o_ref, "bf16")
    check_lse(f64(lse), lse_ref)
    for name, g, gr in zip(("dQ", "dK", "dV"), (dq, dk, dv), oracle.backward(*xs, w.scale, causal)):
        check_grad(f64(g), gr, name)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("B,H,N,d,dt,causal", [(2, 8, 4000, 128, "bf16", True), (1, 8, 3001, 64, "fp16", False)])
def test_ragged_large_every_element(B, H, N, d, dt, causal):
    """A length that is not a multiple of 64 at a size past the tile pipelines' start-up (N = 4000,
    3001): every element of O, lse, dQ, dK and dV against the oracle (per-head pool), with the
    bounds of the full-size parity tests."""
    from oracle_pool import compare_full
    from parity import GRAD_REL_FRO, LSE_MAX, O_MEAN

    ea = require_gpu()
    w = workloads.Workload("ragged_large", B, H, N, d, dt, causal, True, seed=63000 + N + d)
    log(f"ragged large {w}")
    x = workloads.make_inputs(w)
    q, k, v, do = (x[n].cuda() for n in ("q", "k", "v", "do"))
    o, lse = ea.forward(q, k, v, scale=w.scale, causal=causal)
    g = ea.backward(q, k, v, o, lse, do, scale=w.scale, causal=causal)
    torch.cuda.synchronize()
    m = compare_full(w, x, o.cpu(), lse.cpu(), tuple(t.cpu() for t in g))
    log(f"  O max|err| {m['o_max']:.3e} mean {m['o_mean']:.3e}; lse {m['lse_max']:.3e}; "
        f"dq {m['dq_rel_fro']:.3e} dk {m['dk_rel_fro']:.3e} dv {m['dv_rel_fro']:.3e}")
    assert m["finite"] and all(m[n + "_finite"] for n in ("dq", "dk", "dv"))
    assert m["o_over"] == 0, m.get("o_worst_over")
    assert m["o_mean"] <= O_MEAN and m["lse_max"] <= LSE_MAX
    for n in ("dq", "dk", "dv"):
        assert m[n + "_rel_fro"] <= GRAD_REL_FRO, (n, m[n + "_rel_fro"])
