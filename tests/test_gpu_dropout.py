"""Dropout on P (GPU): the library's draws, forward and backward against the oracle.

The oracle (oracle/philox.py) implements the same published generator and
mask layout independently; its generator is pinned to the authors'
known-answer vectors by the CPU tests.  Here:

* attn_dropout_draws equals the oracle's draws byte for byte (integer work:
  bit-exact), for ragged sizes and several seeds and offsets;
* O and lse of attn_fwd_dropout, and dQ, dK, dV of attn_bwd_dropout, match
  the oracle with the same (p, seed, offset) element by element, within the
  tolerances of the tests without dropout (O's scaled by the keep factor,
  which multiplies every rounding error made before it);
* p = 0 gives exactly the results of attn_fwd / attn_bwd, and a different
  seed gives a different O.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from oracle import philox
from oracle_pool import compare_full
from parity import check_grad, check_lse, check_o, f64, log, require_gpu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("BH,Nq,Nk,seed,offset", [
    (1, 1, 1, 0, 0),
    (3, 37, 101, 12345, 0),
    (2, 64, 64, 2**63 + 17, 7),
    (5, 100, 33, 0xDEADBEEFCAFEF00D, 0xFFFFFFFF),
    (1, 300, 257, 42, 1),
])
def test_draws_bit_exact(BH, Nq, Nk, seed, offset):
    ea = require_gpu()
    log(f"dropout draws BH={BH} Nq={Nq} Nk={Nk} seed={seed} offset={offset}")
    got = ea.dropout_draws(BH, Nq, Nk, seed, offset).cpu().numpy()
    for bh in range(BH):
        ref = philox.draws(bh, Nq, Nk, seed, offset)
        bad = np.argwhere(got[bh] != ref)
        assert bad.size == 0, f"head {bh}: {len(bad)} draws differ, first at {bad[:3].tolist()}"


def test_threshold_matches_oracle():
    ea = require_gpu()
    for p in (0.0, 1 / 512, 0.1, 0.25, 0.5, 0.9, 255 / 256):
        assert ea.dropout_threshold(p) == philox.dropout_threshold(p)
    for p in (-0.1, 1.0, float("nan"), 0.001, 0.999):
        with pytest.raises(ValueError):
            philox.dropout_threshold(p)
        with pytest.raises(ValueError):
            ea.dropout_threshold(p)


CASES = [
    # (B, H, N, d, dtype, causal, p, seed, offset)
    (1, 2, 128, 128, "bf16", True, 0.1, 1, 0),
    (2, 2, 256, 64, "bf16", False, 0.2, 77, 3),
    (1, 3, 200, 128, "fp16", True, 0.5, 2**40 + 9, 0),
    (1, 1, 77, 64, "fp16", False, 0.1, 5, 11),
    (2, 1, 333, 128, "bf16", True, 0.3, 123456789, 2),
    (1, 2, 1, 128, "bf16", True, 0.1, 8, 0),
    (1, 2, 512, 128, "bf16", True, 0.9, 31, 0),
]


@pytest.mark.parametrize("B,H,N,d,dt,causal,p,seed,offset", CASES,
                         ids=[f"B{c[0]}H{c[1]}N{c[2]}d{c[3]}{c[4]}{'c' if c[5] else ''}p{c[6]}" for c in CASES])
def test_dropout_forward_backward_match_oracle(B, H, N, d, dt, causal, p, seed, offset):
    ea = require_gpu()
    w = workloads.Workload("drop", B, H, N, d, dt, causal, True, seed=41000 + N + d)
    x = workloads.make_inputs(w)
    q, k, v, do = (x[n].cuda() for n in ("q", "k", "v", "do"))
    log(f"dropout fwd+bwd B={B} H={H} N={N} d={d} {dt} causal={causal} p={p} seed={seed} offset={offset}")
    o, lse = ea.forward_dropout(q, k, v, p, seed, offset, scale=w.scale, causal=causal)
    dq, dk, dv = ea.backward_dropout(q, k, v, o, lse, do, p, seed, offset, scale=w.scale, causal=causal)
    torch.cuda.synchronize()
    args = [workloads.to_f64_numpy(x[n]) for n in ("q", "k", "v")]
    o_ref, lse_ref = oracle.forward(*args, w.scale, causal, dropout=(p, seed, offset))
    eo, _ = check_o(f64(o), o_ref, dt, gain=philox.keep_scale(p))
    el = check_lse(f64(lse), lse_ref)
    grads = oracle.backward(*args, workloads.to_f64_numpy(x["do"]), w.scale, causal, dropout=(p, seed, offset))
    errs = [check_grad(f64(g), gr, name) for name, g, gr in zip(("dQ", "dK", "dV"), (dq, dk, dv), grads)]
    log(f"  max|dO|={eo:.2e} max|dlse|={el:.2e} grads {errs}")


def test_dropout_p_zero_and_seeds():
    ea = require_gpu()
    w = workloads.Workload("drop0", 1, 2, 192, 128, "bf16", True, True, seed=41999)
    x = workloads.make_inputs(w)
    q, k, v, do = (x[n].cuda() for n in ("q", "k", "v", "do"))
    o0, l0 = ea.forward(q, k, v, scale=w.scale, causal=True)
    o1, l1 = ea.forward_dropout(q, k, v, 0.0, 5, 0, scale=w.scale, causal=True)
    g0 = ea.backward(q, k, v, o0, l0, do, scale=w.scale, causal=True)
    g1 = ea.backward_dropout(q, k, v, o1, l1, do, 0.0, 5, 0, scale=w.scale, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(l0, l1)
    for a, b in zip(g0, g1):
        assert torch.equal(a, b)
    o2, l2 = ea.forward_dropout(q, k, v, 0.1, 5, 0, scale=w.scale, causal=True)
    o3, l3 = ea.forward_dropout(q, k, v, 0.1, 6, 0, scale=w.scale, causal=True)
    o4, _ = ea.forward_dropout(q, k, v, 0.1, 5, 0, scale=w.scale, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(l2, l0) and torch.equal(l3, l0)        # lse is the softmax's own
    assert not torch.equal(o2, o3) and torch.equal(o2, o4)     # seeds differ; the same seed repeats


@pytest.mark.timeout(900)
def test_dropout_full_size_headline_every_element():
    """The 4 x 32 x 4096 x 128 causal bf16 workload with p = 0.1, in the launch configuration the
    benchmark's dropout run times: every element of O, lse, dQ, dK and dV against the oracle."""
    ea = require_gpu()
    w = workloads.WORKLOADS[workloads.HEADLINE]
    p, seed = 0.1, 2026
    log(f"dropout full size {w.name} p={p} seed={seed}")
    x = workloads.make_inputs(w)
    q, k, v, do = (x[n].cuda() for n in ("q", "k", "v", "do"))
    o, lse = ea.forward_dropout(q, k, v, p, seed, 0, scale=w.scale, causal=w.causal)
    dq, dk, dv = ea.backward_dropout(q, k, v, o, lse, do, p, seed, 0, scale=w.scale, causal=w.causal)
    torch.cuda.synchronize()
    # sum_j dK_j = 0 holds with dropout too (each row of dS sums to 0)
    sk = dk.double().sum(dim=2).norm(dim=-1)
    assert bool((sk <= 2e-2 * dk.double().norm(dim=(2, 3))).all())
    grads = tuple(g.cpu() for g in (dq, dk, dv))
    m = compare_full(w, x, o.cpu(), lse.cpu(), grads, dropout=(p, seed, 0))
    log(f"  O over {m['o_elements']} elements: max|err| {m['o_max']:.3e} mean|err| {m['o_mean']:.3e} "
        f"rel. Frobenius {m['o_rel_fro']:.3e}; lse max|err| {m['lse_max']:.3e}; rel. Frobenius dq "
        f"{m['dq_rel_fro']:.3e} dk {m['dk_rel_fro']:.3e} dv {m['dv_rel_fro']:.3e}")
    gain = philox.keep_scale(p)
    assert m["finite"] and all(m[g + "_finite"] for g in ("dq", "dk", "dv"))
    assert m["o_over"] == 0, m.get("o_worst_over")
    assert m["o_mean"] <= 1e-3 * gain + m["o_mean_half_ulp"]
    assert m["o_rel_fro"] <= 1e-2
    assert m["lse_max"] <= 1e-3
    for g in ("dq", "dk", "dv"):
        assert m[g + "_rel_fro"] <= 2e-2, (g, m[g + "_rel_fro"])


@pytest.mark.parametrize("N,d,causal", [(200, 128, True), (130, 64, False)])
def test_dropout_token_major_layout(N, d, causal):
    """[B, N, H, d] tensors (as transposed views) through the strided entry points: the mask is that of
    (batch, head, query, key), so the results equal the contiguous call's and match the oracle."""
    ea = require_gpu()
    w = workloads.Workload("drop_nhd", 2, 3, N, d, "bf16", causal, True, seed=42000 + N)
    x = workloads.make_inputs(w)
    p, seed, offset = 0.2, 99, 5
    log(f"dropout token-major B=2 H=3 N={N} d={d} causal={causal}")
    cont = {n: x[n].cuda() for n in ("q", "k", "v", "do")}
    nhd = {n: x[n].transpose(1, 2).contiguous().cuda().transpose(1, 2) for n in ("q", "k", "v", "do")}
    assert not nhd["q"].is_contiguous()
    o1, l1 = ea.forward_dropout(cont["q"], cont["k"], cont["v"], p, seed, offset, scale=w.scale, causal=causal)
    o2, l2 = ea.forward_dropout(nhd["q"], nhd["k"], nhd["v"], p, seed, offset, scale=w.scale, causal=causal)
    g1 = ea.backward_dropout(cont["q"], cont["k"], cont["v"], o1, l1, cont["do"], p, seed, offset, scale=w.scale,
                             causal=causal)
    g2 = ea.backward_dropout(nhd["q"], nhd["k"], nhd["v"], o2, l2, nhd["do"], p, seed, offset, scale=w.scale,
                             causal=causal)
    torch.cuda.synchronize()
    assert o2.stride() == nhd["q"].stride()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    args = [workloads.to_f64_numpy(x[n]) for n in ("q", "k", "v")]
    o_ref, lse_ref = oracle.forward(*args, w.scale, causal, dropout=(p, seed, offset))
    check_o(f64(o2), o_ref, "bf16", gain=philox.keep_scale(p))
    check_lse(f64(l2), lse_ref)
    grads = oracle.backward(*args, workloads.to_f64_numpy(x["do"]), w.scale, causal, dropout=(p, seed, offset))
    for name, a, b, gr in zip(("dQ", "dK", "dV"), g1, g2, grads):
        check_grad(f64(b), gr, name)
        assert torch.equal(a, b), f"{name}: token-major result differs from the contiguous one"


def test_dropout_extreme_probability():
    """p = 255/256 (t = 255, keep factor 256): rows whose visible keys are all dropped give O = 0 exactly,
    the rest match the oracle, and the gradients stay finite and match."""
    ea = require_gpu()
    w = workloads.Workload("drop_hi", 1, 2, 300, 64, "bf16", True, True, seed=43001)
    x = workloads.make_inputs(w)
    q, k, v, do = (x[n].cuda() for n in ("q", "k", "v", "do"))
    p, seed = 255 / 256, 3
    assert philox.dropout_threshold(p) == 255
    log("dropout p=255/256 B=1 H=2 N=300 d=64 causal")
    o, lse = ea.forward_dropout(q, k, v, p, seed, 0, scale=w.scale, causal=True)
    dq, dk, dv = ea.backward_dropout(q, k, v, o, lse, do, p, seed, 0, scale=w.scale, causal=True)
    torch.cuda.synchronize()
    args = [workloads.to_f64_numpy(x[n]) for n in ("q", "k", "v")]
    o_ref, lse_ref = oracle.forward(*args, w.scale, True, dropout=(p, seed, 0))
    n_zero = 0
    for h in range(2):
        keep = np.tril(philox.keep_mask(h, 300, 300, p, seed, 0))
        empty = ~keep.any(axis=1)
        n_zero += int(empty.sum())
        assert (o[0, h][torch.from_numpy(empty).cuda()] == 0).all().item()
    assert n_zero > 0
    check_o(f64(o), o_ref, "bf16", gain=philox.keep_scale(p))
    check_lse(f64(lse), lse_ref)
    grads = oracle.backward(*args, workloads.to_f64_numpy(x["do"]), w.scale, True, dropout=(p, seed, 0))
    for name, g, gr in zip(("dQ", "dK", "dV"), (dq, dk, dv), grads):
        check_grad(f64(g), gr, name)
