"""Seeded random shapes against the fp64 oracle (GPU).

Forty forward+backward cases and thirty KV-cache cases drawn from a fixed
seed: batch and head counts, any sequence length up to 700 (so most are not
multiples of the tile sizes), both head dimensions, both dtypes, causal or
not, contiguous or token-major [B, N, H, d] tensors, and for the KV-cache
calls any Nq <= Nk and a random split count.  Every element is compared.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
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
