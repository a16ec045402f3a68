"""The whole-tensor comparison used at full size, checked on the CPU.

Feeding it the oracle's own result rounded to the output format must give
errors at the rounding floor and no element over its bound; a single
planted wrong element must be counted and located; a wrong gradient head
must raise the whole-tensor relative Frobenius error by the amount that head
carries.  The rounding helper must agree with torch's own round to nearest
even.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from oracle_pool import compare_full, round_to


def _rounded(a: np.ndarray, dt: torch.dtype) -> torch.Tensor:
    return torch.from_numpy(a).to(dt)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_round_to_matches_torch(dtype):
    rng = np.random.default_rng(3)
    x = rng.standard_normal(10000) * np.exp2(rng.integers(-8, 8, 10000))
    dt = torch.bfloat16 if dtype == "bf16" else torch.float16
    ref = torch.from_numpy(x.astype(np.float32)).to(dt).double().numpy()
    assert np.array_equal(round_to(x.astype(np.float32).astype(np.float64), dtype), ref)


def test_compare_full_rounding_floor_and_planted_errors():
    w = workloads.Workload("pool", 2, 3, 96, 16, "bf16", True, True, seed=4242)
    x = workloads.make_inputs(w)
    a = {n: workloads.to_f64_numpy(x[n]) for n in ("q", "k", "v", "do")}
    o_ref, lse_ref = oracle.forward(a["q"], a["k"], a["v"], w.scale, True)
    g_ref = oracle.backward(a["q"], a["k"], a["v"], a["do"], w.scale, True)
    o = _rounded(o_ref, torch.bfloat16)
    lse = torch.from_numpy(lse_ref.astype(np.float32))
    grads = tuple(_rounded(g, torch.bfloat16) for g in g_ref)

    m = compare_full(w, x, o, lse, grads, workers=2)
    assert m["heads"] == 6 and m["o_elements"] == o_ref.size
    assert m["o_over"] == 0 and m["finite"]
    assert m["o_max"] <= m["o_floor"] + 1e-15 and m["o_mean"] < 1e-3
    assert m["lse_max"] < 1e-5
    for g in ("dq", "dk", "dv"):
        assert m[g + "_rel_fro"] < 4e-3

    o_bad = o.clone()
    o_bad[1, 2, 17, 5] += 0.05
    dk_bad = grads[1].clone()
    dk_bad[0, 1] *= 1.5
    m2 = compare_full(w, x, o_bad, lse, (grads[0], dk_bad, grads[2]), workers=2)
    assert m2["o_over"] == 1
    assert m2["o_worst_over"][:4] == (1, 2, 17, 5)
    fro_head = np.linalg.norm(g_ref[1][0, 1]) / np.linalg.norm(g_ref[1])
    assert m2["dk_rel_fro"] == pytest.approx(0.5 * fro_head, rel=2e-2)
    assert m2["dk_worst_head"] == pytest.approx(0.5, rel=2e-2)


def test_compare_full_passes_the_alibi_slopes_to_every_head():
    """With per-head slopes the workers must evaluate the biased oracle: the
    oracle's own biased result matches at the rounding floor, and the same
    result compared without the slopes does not."""
    w = workloads.Workload("pool_alibi", 2, 3, 80, 16, "bf16", True, True, seed=4243)
    x = workloads.make_inputs(w)
    a = {n: workloads.to_f64_numpy(x[n]) for n in ("q", "k", "v", "do")}
    slopes = np.array([0.5, 0.25, 0.125])
    o_ref, lse_ref = oracle.forward(a["q"], a["k"], a["v"], w.scale, True, alibi_slopes=slopes)
    g_ref = oracle.backward(a["q"], a["k"], a["v"], a["do"], w.scale, True, alibi_slopes=slopes)
    o = _rounded(o_ref, torch.bfloat16)
    lse = torch.from_numpy(lse_ref.astype(np.float32))
    grads = tuple(_rounded(g, torch.bfloat16) for g in g_ref)
    m = compare_full(w, x, o, lse, grads, workers=2, alibi_slopes=slopes)
    assert m["o_over"] == 0 and m["o_max"] <= m["o_floor"] + 1e-15 and m["lse_max"] < 1e-5
    for g in ("dq", "dk", "dv"):
        assert m[g + "_rel_fro"] < 4e-3
    m_plain = compare_full(w, x, o, lse, grads, workers=2)
    assert m_plain["o_over"] > 0 and m_plain["lse_max"] > 1e-2
