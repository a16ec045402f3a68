"""Seeded random shapes against the fp64 oracle (GPU).

Forty forward+backward cases and thirty KV-cache cases drawn from a fixed
seed: batch and head counts, any sequence length up to 700 (so most are not
multiples of the tile sizes), both head dimensions, both dtypes, causal or
not, contiguous or token-major [B, N, H, d] tensors, and for the KV-cache
calls any Nq <= Nk and a random split count.  Fifteen more forward+backward
cases with dropout (random probability, seed and offset) come from their own
generator, so the cases above are unchanged.  Every element is compared.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from oracle import philox
from parity import check_grad, check_lse, check_o, f64, log, require_gpu

pytestmark = pytest.mark.gpu

_rng = np.random.default_rng(20261202)
TRAIN = [dict(B=int(_rng.integers(1, 3)), H=int(_rng.integers(1, 4)), N=int(_rng.integers(1, 701)),
              d=int(_rng.choice([64, 128])), dt=str(_rng.choice(["bf16", "fp16"])), causal=bool(_rng.integers(0, 2)),
              nhd=bool(_rng.integers(0, 2)), seed=int(_rng.integers(1 << 30))) for _ in range(40)]
KV = []
for _ in range(30):
    nq = int(_rng.integers(1, 71))
    KV.append(dict(B=int(_rng.integers(1, 3)), H=int(_rng.integers(1, 5)), Nq=nq, Nk=int(_rng.integers(nq, 3001)),
                   d=int(_rng.choice([64, 128])), dt=str(_rng.choice(["bf16", "fp16"])),
                   causal=bool(_rng.integers(0, 2)), splits=int(_rng.choice([0, 0, 1, 3, 17, 200])),
                   seed=int(_rng.integers(1 << 30))))


def _id(c):
    return "-".join(f"{k}{v}" for k, v in c.items() if k != "seed")


@pytest.mark.parametrize("c", TRAIN, ids=[_id(c) for c in TRAIN])
def test_random_forward_backward(c):
    ea = require_gpu()
    w = workloads.Workload("rand", c["B"], c["H"], c["N"], c["d"], c["dt"], c["causal"], True, seed=c["seed"])
    x = workloads.make_inputs(w)
    log(f"random fwd+bwd {_id(c)}")
    if c["nhd"]:
        dev = {n: x[n].transpose(1, 2).contiguous().cuda().transpose(1, 2) for n in ("q", "k", "v", "do")}
    else:
        dev = {n: x[n].cuda() for n in ("q", "k", "v", "do")}
    o, lse = ea.forward(dev["q"], dev["k"], dev["v"], scale=w.scale, causal=w.causal)
    dq, dk, dv = ea.backward(dev["q"], dev["k"], dev["v"], o, lse, dev["do"], scale=w.scale, causal=w.causal)
    torch.cuda.synchronize()
    args = [workloads.to_f64_numpy(x[n]) for n in ("q", "k", "v")]
    o_ref, lse_ref = oracle.forward(*args, w.scale, w.causal)
    check_o(f64(o), o_ref, w.dtype)
    check_lse(f64(lse), lse_ref)
    grads = oracle.backward(*args, workloads.to_f64_numpy(x["do"]), w.scale, w.causal)
    for name, g, gr in zip(("dQ", "dK", "dV"), (dq, dk, dv), grads):
        check_grad(f64(g), gr, name)


@pytest.mark.parametrize("c", KV, ids=[_id(c) for c in KV])
def test_random_kvcache(c):
    ea = require_gpu()
    w = workloads.KvWorkload("rand_kv", c["B"], c["H"], c["Nq"], c["Nk"], c["d"], c["dt"], c["causal"], seed=c["seed"])
    x = workloads.make_kv_inputs(w)
    q, k, v = (x[n].cuda() for n in ("q", "k", "v"))
    log(f"random kvcache {_id(c)}")
    o, lse = ea.forward_kvcache(q, k, v, scale=w.scale, causal=w.causal, num_splits=c["splits"])
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.forward(*(workloads.to_f64_numpy(x[n]) for n in ("q", "k", "v")), w.scale, w.causal)
    check_o(f64(o), o_ref, w.dtype)
    check_lse(f64(lse), lse_ref)


_rng_d = np.random.default_rng(20261203)
DROP = [dict(B=int(_rng_d.integers(1, 3)), H=int(_rng_d.integers(1, 4)), N=int(_rng_d.integers(1, 701)),
             d=int(_rng_d.choice([64, 128])), dt=str(_rng_d.choice(["bf16", "fp16"])),
             causal=bool(_rng_d.integers(0, 2)), p=float(_rng_d.choice([0.05, 0.1, 0.2, 0.5])),
             dseed=int(_rng_d.integers(1 << 62)), offset=int(_rng_d.integers(1 << 32)),
             seed=int(_rng_d.integers(1 << 30))) for _ in range(15)]


@pytest.mark.parametrize("c", DROP, ids=[_id(c) for c in DROP])
def test_random_dropout_forward_backward(c):
    ea = require_gpu()
    w = workloads.Workload("rand_drop", c["B"], c["H"], c["N"], c["d"], c["dt"], c["causal"], True, seed=c["seed"])
    x = workloads.make_inputs(w)
    q, k, v, do = (x[n].cuda() for n in ("q", "k", "v", "do"))
    log(f"random dropout fwd+bwd {_id(c)}")
    o, lse = ea.forward_dropout(q, k, v, c["p"], c["dseed"], c["offset"], scale=w.scale, causal=w.causal)
    dq, dk, dv = ea.backward_dropout(q, k, v, o, lse, do, c["p"], c["dseed"], c["offset"], scale=w.scale,
                                     causal=w.causal)
    torch.cuda.synchronize()
    drop = (c["p"], c["dseed"], c["offset"])
    args = [workloads.to_f64_numpy(x[n]) for n in ("q", "k", "v")]
    o_ref, lse_ref = oracle.forward(*args, w.scale, w.causal, dropout=drop)
    check_o(f64(o), o_ref, w.dtype, gain=philox.keep_scale(c["p"]))
    check_lse(f64(lse), lse_ref)
    grads = oracle.backward(*args, workloads.to_f64_numpy(x["do"]), w.scale, w.causal, dropout=drop)
    for name, g, gr in zip(("dQ", "dK", "dV"), (dq, dk, dv), grads):
        check_grad(f64(g), gr, name)
