"""Very long sequences (GPU): offsets and grid sizes far past the training workloads.

A 262144-token causal head and a decoding step against a cache of 2^20
positions (every output row against the oracle).  For the long head the
oracle evaluates what it can without the whole N x N product: O, lse and dQ
of sampled query rows (a row's values depend on that row alone), and dK, dV
of the last 64 keys (under the causal mask only the last 64 query rows reach
them); the backward is also checked by invariants over every key.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import check_grad, check_lse, check_o, f64, log, require_gpu, sample_rows

pytestmark = pytest.mark.gpu


def test_long_sequence_sampled_rows_key_tail_and_invariants():
    ea = require_gpu()
    w = workloads.Workload("long", 1, 1, 1 << 18, 128, "bf16", True, True, seed=71001)
    x = workloads.make_inputs(w)
    q, k, v, do = (x[n].cuda() for n in ("q", "k", "v", "do"))
    log(f"long sequence N={w.N} d={w.d} causal bf16: forward")
    o, lse = ea.forward(q, k, v, scale=w.scale, causal=True)
    torch.cuda.synchronize()
    rows = sample_rows(w.N, 48, seed=71002)
    qh, kh, vh = (workloads.to_f64_numpy(x[n][0, 0]) for n in ("q", "k", "v"))
    o_ref, lse_ref = oracle.forward_head_rows(qh, kh, vh, w.scale, True, rows)
    eo, _ = check_o(f64(o[0, 0][rows]), o_ref, "bf16")
    el = check_lse(f64(lse[0, 0][rows]), lse_ref)
    log(f"  {len(rows)} rows: O max|err| {eo:.2e}, lse max|err| {el:.2e}")
    log("  backward")
    dq, dk, dv = ea.backward(q, k, v, o, lse, do, scale=w.scale, causal=True)
    torch.cuda.synchronize()
    for t in (dq, dk, dv):
        assert torch.isfinite(t).all().item()
    # softmax shift invariance: the rows of dS sum to 0, so sum_j dK_j = 0;
    # and sum_j dV_j = sum_i dO_i (each row of P sums to 1)
    sk = dk[0, 0].double().sum(0).norm().item()
    nk = dk[0, 0].double().norm().item()
    sv = (dv[0, 0].double().sum(0) - do[0, 0].double().sum(0)).norm().item()
    nv = dv[0, 0].double().norm().item()
    log(f"  |sum dK| / |dK| = {sk / nk:.2e}, |sum dV - sum dO| / |dV| = {sv / nv:.2e}")
    assert sk <= 2e-2 * nk and sv <= 2e-2 * nv
    doh = workloads.to_f64_numpy(x["do"][0, 0])
    dq_ref, _, _ = oracle.attention.backward_head_rows(qh, kh, vh, doh, w.scale, True, rows)
    e = check_grad(f64(dq[0, 0][rows]), dq_ref, "dQ (sampled rows)")
    log(f"  dQ of {len(rows)} rows: relative Frobenius error {e:.2e}")
    j0 = w.N - 64
    _, dk_ref, dv_ref = oracle.attention.backward_head_rows(qh, kh, vh, doh, w.scale, True, np.arange(j0, w.N))
    ek = check_grad(f64(dk[0, 0][j0:]), dk_ref[j0:], "dK (last 64 keys)")
    ev = check_grad(f64(dv[0, 0][j0:]), dv_ref[j0:], "dV (last 64 keys)")
    log(f"  dK, dV of the last 64 keys: relative Frobenius errors {ek:.2e}, {ev:.2e}")


def test_decode_against_a_million_positions():
    ea = require_gpu()
    w = workloads.KvWorkload("long_kv", 1, 2, 2, 1 << 20, 128, "bf16", True, seed=71003)
    x = workloads.make_kv_inputs(w)
    q, k, v = (x[n].cuda() for n in ("q", "k", "v"))
    splits = ea.attn_fwd_kvcache_splits(w.B, w.H, w.Nq, w.Nk, w.d, 0)
    log(f"decode Nq={w.Nq} Nk={w.Nk} ({splits} splits)")
    o, lse = ea.forward_kvcache(q, k, v, scale=w.scale, causal=True)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.forward(*(workloads.to_f64_numpy(x[n]) for n in ("q", "k", "v")), w.scale, True)
    eo, _ = check_o(f64(o), o_ref, "bf16")
    el = check_lse(f64(lse), lse_ref)
    log(f"  O max|err| {eo:.2e}, lse max|err| {el:.2e}")
