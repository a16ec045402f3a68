"""Both forward launch shapes on every kind of forward call (runs on the GPU).

The forward runs either 8-wave workgroups of 256 queries or 4-wave workgroups
of 128 queries, chosen per call from N, d and causal.  Both give every wave
the same 32 query rows and walk its keys in the same 32-key blocks in the
same order, so their O and lse must agree bit for bit.  Each case below runs
with the shape forced both ways (ATTN_FWD_WAVES, read by the library on every
call): the two results must be identical, and the 8-wave one, which the
automatic choice no longer takes at these lengths, is compared with the fp64
oracle over every element.  The cases cover both head sizes, causal and not,
lengths with and without a partial last tile, and the plain, token-major
(strided), ALiBi and dropout forms.
"""
import os

import numpy as np
import pytest
import torch

import oracle
import workloads
from oracle import philox
from parity import check_lse, check_o, f64, log, require_gpu

pytestmark = pytest.mark.gpu

CASES = [
    # (B, H, N, d, dtype, causal, form)
    (1, 2, 1000, 128, "bf16", True, "plain"),
    (1, 2, 1000, 128, "fp16", False, "plain"),
    (1, 2, 1024, 128, "bf16", False, "plain"),
    (2, 2, 640, 64, "bf16", True, "plain"),
    (1, 3, 321, 64, "fp16", False, "plain"),
    (1, 2, 65, 128, "bf16", True, "plain"),
    (2, 3, 1000, 128, "bf16", True, "strided"),
    (1, 4, 333, 64, "bf16", False, "strided"),
    (1, 4, 1000, 128, "bf16", True, "alibi"),
    (2, 2, 300, 64, "fp16", False, "alibi"),
    (1, 2, 1000, 128, "bf16", True, "dropout"),
    (1, 2, 500, 64, "fp16", False, "dropout"),
]
DROP_P, DROP_SEED, DROP_OFFSET = 0.1, 77, 3


def _id(c):
    B, H, N, d, dt, causal, form = c
    return f"{form}-B{B}H{H}N{N}d{d}{dt}{'causal' if causal else ''}"


def _slopes(H):
    return torch.tensor([2.0 ** (-8.0 * (h + 1) / H) for h in range(H)], dtype=torch.float32)


def _forward(ea, form, q, k, v, w):
    if form == "alibi":
        return ea.forward_alibi(q, k, v, _slopes(w.H).cuda(), scale=w.scale, causal=w.causal)
    if form == "dropout":
        return ea.forward_dropout(q, k, v, DROP_P, DROP_SEED, DROP_OFFSET, scale=w.scale, causal=w.causal)
    if form == "strided":
        # token-major [B, N, H, d] storage seen as [B, H, N, d] views
        q, k, v = (t.transpose(1, 2).contiguous().transpose(1, 2) for t in (q, k, v))
        assert not q.is_contiguous()
    return ea.forward(q, k, v, scale=w.scale, causal=w.causal)


@pytest.mark.parametrize("c", CASES, ids=[_id(c) for c in CASES])
def test_both_forward_shapes_bitwise_equal_and_match_the_oracle(c, monkeypatch):
    ea = require_gpu()
    B, H, N, d, dt, causal, form = c
    w = workloads.Workload("shapes", B, H, N, d, dt, causal, False, seed=64000 + 3 * N + d + B + H)
    log(f"forward shapes {form} {w}")
    x = workloads.make_inputs(w)
    q, k, v = (x[n].cuda() for n in ("q", "k", "v"))
    out = {}
    for waves in ("4", "8"):
        monkeypatch.setenv("ATTN_FWD_WAVES", waves)
        out[waves] = _forward(ea, form, q, k, v, w)
        torch.cuda.synchronize()
    monkeypatch.delenv("ATTN_FWD_WAVES")
    (o4, l4), (o8, l8) = out["4"], out["8"]
    assert torch.equal(o4, o8), f"O differs between the shapes: max {float((o4.float() - o8.float()).abs().max())}"
    assert torch.equal(l4, l8), f"lse differs between the shapes: max {float((l4 - l8).abs().max())}"
    args = [workloads.to_f64_numpy(x[n]) for n in ("q", "k", "v")]
    kw, gain = {}, 1.0
    if form == "alibi":
        kw["alibi_slopes"] = _slopes(H).double().numpy()
    if form == "dropout":
        kw["dropout"] = (DROP_P, DROP_SEED, DROP_OFFSET)
        gain = philox.keep_scale(DROP_P)
    o_ref, lse_ref = oracle.forward(*args, w.scale, causal, **kw)
    eo, mo = check_o(f64(o8), o_ref, dt, gain=gain)
    el = check_lse(f64(l8), lse_ref)
    log(f"  O max {eo:.2e} mean {mo:.2e}, lse max {el:.2e}")


def test_automatic_shape_equals_both_forced_shapes(monkeypatch):
    """Without the variable the library picks a shape by itself; at the
    headline size (B=4, H=32, N=4096, d=128, causal) its O and lse equal
    those of both forced shapes bit for bit."""
    ea = require_gpu()
    w = workloads.WORKLOADS[workloads.HEADLINE].with_size(backward=False)
    x = workloads.make_inputs(w)
    q, k, v = (x[n].cuda() for n in ("q", "k", "v"))
    monkeypatch.delenv("ATTN_FWD_WAVES", raising=False)
    o, lse = ea.forward(q, k, v, scale=w.scale, causal=True)
    for waves in ("4", "8"):
        monkeypatch.setenv("ATTN_FWD_WAVES", waves)
        o2, l2 = ea.forward(q, k, v, scale=w.scale, causal=True)
        torch.cuda.synchronize()
        assert torch.equal(o, o2) and torch.equal(lse, l2), f"ATTN_FWD_WAVES={waves} differs from the default"
    assert os.environ.get("ATTN_FWD_WAVES") == "8"
    assert np.isfinite(f64(lse)).all()
