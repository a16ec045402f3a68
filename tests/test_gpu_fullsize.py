"""Parity over every element at the full workload sizes (runs on the GPU).

Each workload runs once through the C ABI in the configuration the benchmark
times (forward, then the backward on the GPU's own O and lse, as in
training); the fp64 oracle then evaluates every (batch, head) in a pool of
host processes and the errors are taken over the whole tensors:
O max|err| <= 1e-2 (half an output ulp + 1e-3 where |O_ref| >= 4) and
mean|err| <= 1e-3 over all B*H*N*d elements, lse max|err| <= 1e-3 over all
rows, and ||G - G_ref||_F / ||G_ref||_F <= 2e-2 over each whole gradient.
The gradient invariants sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i are
checked on every head as well.
"""
import pytest
import torch

import workloads
from oracle_pool import compare_full
from parity import GRAD_REL_FRO, LSE_MAX, O_MEAN, log, require_gpu

pytestmark = pytest.mark.gpu


def _invariants(dk, dv, do, what):
    """Rows of dS sum to 0, so sum_j dK_j = 0; rows of P sum to 1, so
    sum_j dV_j = sum_i dO_i.  Per head, relative to the head's Frobenius norm
    (each of the N summed values carries its own rounding)."""
    sk = dk.double().sum(dim=2).norm(dim=-1)
    nk = dk.double().norm(dim=(2, 3))
    assert bool((sk <= 2e-2 * nk).all()), f"{what}: |sum_j dK_j| / |dK| = {(sk / nk).max().item():.3e}"
    sv = (dv.double().sum(dim=2) - do.double().sum(dim=2)).norm(dim=-1)
    nv = dv.double().norm(dim=(2, 3))
    assert bool((sv <= 2e-2 * nv).all()), f"{what}: |sum dV - sum dO| / |dV| = {(sv / nv).max().item():.3e}"


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", list(workloads.WORKLOADS))
def test_every_element_at_full_size(name):
    ea = require_gpu()
    w = workloads.WORKLOADS[name]
    log(f"full size {w.name}: B={w.B} H={w.H} N={w.N} d={w.d} {w.dtype} causal={w.causal} "
        f"backward={w.backward} seed={w.seed}")
    x = workloads.make_inputs(w)
    q, k, v = (x[n].cuda() for n in ("q", "k", "v"))
    o, lse = ea.forward(q, k, v, scale=w.scale, causal=w.causal)
    grads = None
    if w.backward:
        do = x["do"].cuda()
        grads = ea.backward(q, k, v, o, lse, do, scale=w.scale, causal=w.causal)
        torch.cuda.synchronize()
        _invariants(grads[1], grads[2], do, w.name)
        grads = tuple(g.cpu() for g in grads)
        del do
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu()
    del q, k, v
    m = compare_full(w, x, o, lse, grads)
    line = (f"  {w.name}: {m['heads']} heads on {m['workers']} workers; O over {m['o_elements']} elements: "
            f"max|err| {m['o_max']:.3e} mean|err| {m['o_mean']:.3e} (|O_ref|>=4: {m['o_big']} elements, "
            f"oracle rounding floor {m['o_floor']:.3e}); lse max|err| {m['lse_max']:.3e}")
    if grads is not None:
        line += "; rel. Frobenius " + " ".join(
            f"{g} {m[g + '_rel_fro']:.3e} (worst head {m[g + '_worst_head']:.3e})" for g in ("dq", "dk", "dv"))
    log(line)
    assert m["finite"], "non-finite O or lse"
    assert m["o_over"] == 0, f"{m['o_over']} O elements over their bound; first (b, h, row, col, gpu, ref): " \
                             f"{m.get('o_worst_over')}"
    assert m["o_mean"] <= O_MEAN, f"O mean|err| {m['o_mean']:.3e} > {O_MEAN}"
    assert m["lse_max"] <= LSE_MAX, f"lse max|err| {m['lse_max']:.3e} > {LSE_MAX}"
    if grads is not None:
        for g in ("dq", "dk", "dv"):
            assert m[g + "_finite"], f"non-finite {g}"
            assert m[g + "_rel_fro"] <= GRAD_REL_FRO, f"{g}: relative Frobenius error {m[g + '_rel_fro']:.3e}"
