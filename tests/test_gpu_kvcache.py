"""Parity of the KV-cache forward (Nq queries against Nk cached keys) with the fp64 oracle (GPU).

attn_fwd_kvcache splits the key axis into ranges, one wave each, and merges
the ranges' softmax states.  The result must match the oracle's plain
definition with the bottom-right causal mask (query i sees keys
j <= i + Nk - Nq) for every split count, including counts that leave some
ranges empty under the causal mask.  Every element is compared: the oracle
row for one query costs one pass over Nk keys, so even the full-size
decoding workloads are checked in whole.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import check_lse, check_o, f64, log, require_gpu

pytestmark = pytest.mark.gpu

CASES = [
    # (B, H, Nq, Nk, d, dtype, causal, num_splits, qk_gain)
    (1, 2, 1, 1, 64, "bf16", True, 0, 1.0),
    (2, 3, 1, 300, 128, "bf16", True, 0, 1.0),
    (1, 2, 1, 4096, 128, "fp16", False, 0, 1.0),
    (2, 2, 5, 1000, 64, "bf16", True, 0, 1.0),
    (1, 2, 32, 777, 128, "bf16", True, 7, 1.0),
    (1, 1, 40, 100, 64, "fp16", True, 0, 1.0),
    (1, 1, 40, 100, 128, "bf16", True, 100, 1.0),     # 32-key splits: the first query block's last split is empty
    (1, 2, 64, 64, 128, "bf16", True, 0, 1.0),        # square: the attn_fwd mask
    (1, 2, 70, 50, 64, "bf16", False, 3, 1.0),        # non-causal, more queries than keys
    (2, 4, 8, 2048, 128, "bf16", True, 1, 1.0),       # one split: no merge across ranges
    (1, 2, 3, 5000, 128, "bf16", True, 0, 2.0),       # peaky rows (Q and K x2)
    (1, 2, 16, 33, 64, "fp16", True, 2, 1.0),
]


def _ids(c):
    B, H, Nq, Nk, d, dt, causal, sp, g = c
    return f"B{B}H{H}q{Nq}k{Nk}d{d}{dt}{'causal' if causal else ''}s{sp}" + ("x2" if g != 1.0 else "")


def _run_and_check(ea, w, num_splits, guard=0):
    x = workloads.make_kv_inputs(w)
    q, k, v = (x[n].cuda() for n in ("q", "k", "v"))
    log(f"kvcache {w.name}: B={w.B} H={w.H} Nq={w.Nq} Nk={w.Nk} d={w.d} {w.dtype} causal={w.causal} "
        f"splits={ea.attn_fwd_kvcache_splits(w.B, w.H, w.Nq, w.Nk, w.d, num_splits)}")
    if guard:
        # B = H = 1: outputs at the start of NaN-filled buffers, to show stores past row Nq - 1
        assert w.B == 1 and w.H == 1
        ob = torch.full((1, 1, w.Nq + guard, w.d), float("nan"), dtype=q.dtype, device="cuda")
        lb = torch.full((1, 1, w.Nq + guard), float("nan"), dtype=torch.float32, device="cuda")
        o, lse = ob[:, :, :w.Nq], lb[:, :, :w.Nq]
        ws = torch.empty(ea.attn_fwd_kvcache_workspace_bytes(1, 1, w.Nq, w.Nk, w.d, num_splits), dtype=torch.uint8,
                         device="cuda")
        ea.attn_fwd_kvcache(q, k, v, o, lse, w.scale, w.causal, ws, num_splits)
    else:
        o, lse = ea.forward_kvcache(q, k, v, scale=w.scale, causal=w.causal, num_splits=num_splits)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.forward(*(workloads.to_f64_numpy(x[n]) for n in ("q", "k", "v")), w.scale, w.causal)
    eo, _ = check_o(f64(o), o_ref, w.dtype)
    el = check_lse(f64(lse), lse_ref)
    if guard:
        assert torch.isnan(ob[:, :, w.Nq:]).all() and torch.isnan(lb[:, :, w.Nq:]).all(), "store past row Nq - 1"
    log(f"  max|dO|={eo:.2e} max|dlse|={el:.2e}")
    return o, lse


@pytest.mark.parametrize("B,H,Nq,Nk,d,dt,causal,splits,gain", CASES, ids=[_ids(c) for c in CASES])
def test_kvcache_matches_oracle(B, H, Nq, Nk, d, dt, causal, splits, gain):
    ea = require_gpu()
    w = workloads.KvWorkload("kv", B, H, Nq, Nk, d, dt, causal, seed=31000 + 13 * Nk + Nq + d, qk_gain=gain)
    _run_and_check(ea, w, splits)


@pytest.mark.parametrize("splits", [1, 2, 5, 0, 4096])
def test_kvcache_split_counts_and_guard_rows(splits):
    ea = require_gpu()
    w = workloads.KvWorkload("kv_guard", 1, 1, 37, 1111, 128, "bf16", True, seed=32001)
    _run_and_check(ea, w, splits, guard=64)


def test_kvcache_square_agrees_with_attn_fwd():
    """With Nq == Nk both entry points compute the same causal attention."""
    ea = require_gpu()
    w = workloads.Workload("sq", 2, 2, 320, 128, "bf16", True, False, seed=32002)
    x = workloads.make_inputs(w)
    q, k, v = (x[n].cuda() for n in ("q", "k", "v"))
    o1, l1 = ea.forward(q, k, v, scale=w.scale, causal=True)
    o2, l2 = ea.forward_kvcache(q, k, v, scale=w.scale, causal=True)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.forward(*(workloads.to_f64_numpy(x[n]) for n in ("q", "k", "v")), w.scale, True)
    for o, lse in ((o1, l1), (o2, l2)):
        check_o(f64(o), o_ref, "bf16")
        check_lse(f64(lse), lse_ref)
    assert float((o1.float() - o2.float()).abs().max()) <= 2e-2


@pytest.mark.parametrize("name", sorted(n for n, w in workloads.KV_WORKLOADS.items() if w.kv_heads == w.H))
def test_kvcache_full_size_workloads(name):
    """The decoding workloads at full size, in the launch configuration the benchmark times."""
    ea = require_gpu()
    w = workloads.KV_WORKLOADS[name]
    assert ea.attn_fwd_kvcache_splits(w.B, w.H, w.Nq, w.Nk, w.d, 0) > 1
    _run_and_check(ea, w, 0)


@pytest.mark.parametrize("name", sorted(n for n, w in workloads.KV_WORKLOADS.items() if w.kv_heads != w.H))
def test_kvcache_full_size_grouped_workloads(name):
    """Grouped-head decoding workloads at full size (every element against the oracle with K, V repeated)."""
    ea = require_gpu()
    w = workloads.KV_WORKLOADS[name]
    x = workloads.make_kv_inputs(w)
    G = w.H // w.kv_heads
    log(f"kvcache {w.name}: B={w.B} H={w.H} Hkv={w.kv_heads} Nq={w.Nq} Nk={w.Nk}")
    o, lse = ea.forward_kvcache_gqa(x["q"].cuda(), x["k"].cuda(), x["v"].cuda(), scale=w.scale, causal=w.causal)
    torch.cuda.synchronize()
    k_rep = np.repeat(workloads.to_f64_numpy(x["k"]), G, axis=1)
    v_rep = np.repeat(workloads.to_f64_numpy(x["v"]), G, axis=1)
    o_ref, lse_ref = oracle.forward(workloads.to_f64_numpy(x["q"]), k_rep, v_rep, w.scale, w.causal)
    eo, _ = check_o(f64(o), o_ref, w.dtype)
    el = check_lse(f64(lse), lse_ref)
    log(f"  max|dO|={eo:.2e} max|dlse|={el:.2e}")


GQA_CASES = [
    # (B, Hq, Hkv, Nq, Nk, d, dtype, causal, num_splits, alibi)
    (2, 8, 2, 1, 3000, 128, "bf16", True, 0, False),
    (1, 32, 8, 1, 4096, 128, "bf16", True, 0, False),     # 32 query heads on 8 KV heads
    (1, 8, 1, 5, 1000, 64, "fp16", True, 0, False),       # one KV head: 40 (head, query) rows, two tiles
    (2, 6, 3, 7, 700, 128, "bf16", False, 3, False),
    (1, 32, 1, 2, 2048, 128, "bf16", True, 0, True),      # ALiBi slopes per query head
    (1, 4, 4, 3, 500, 64, "bf16", True, 0, False),        # groups of one
    (1, 16, 2, 40, 333, 128, "fp16", True, 0, False),     # 320 rows per KV head, causal rows of many positions
]


@pytest.mark.parametrize("B,Hq,Hkv,Nq,Nk,d,dt,causal,splits,alibi", GQA_CASES,
                         ids=[f"B{c[0]}q{c[1]}kv{c[2]}n{c[3]}k{c[4]}d{c[5]}{c[6]}{'c' if c[7] else ''}s{c[8]}"
                              f"{'alibi' if c[9] else ''}" for c in GQA_CASES])
def test_kvcache_grouped_heads(B, Hq, Hkv, Nq, Nk, d, dt, causal, splits, alibi):
    """Grouped heads: each query head attends with its group's K and V (the oracle repeats them per head)."""
    ea = require_gpu()
    g = torch.Generator(device="cpu")
    g.manual_seed(33000 + Nk + Hq + Nq)
    tdt = {"bf16": torch.bfloat16, "fp16": torch.float16}[dt]
    q = torch.randn((B, Hq, Nq, d), generator=g).to(tdt)
    k = torch.randn((B, Hkv, Nk, d), generator=g).to(tdt)
    v = torch.randn((B, Hkv, Nk, d), generator=g).to(tdt)
    scale = ea.default_scale(d)
    sl = torch.tensor([2.0 ** (-8.0 * (h + 1) / Hq) for h in range(Hq)], dtype=torch.float32) if alibi else None
    log(f"kvcache grouped heads B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} {dt} causal={causal} "
        f"splits={ea.attn_fwd_kvcache_splits(B, Hkv, (Hq // Hkv) * Nq, Nk, d, splits)}")
    o, lse = ea.forward_kvcache_gqa(q.cuda(), k.cuda(), v.cuda(), scale=scale, causal=causal, num_splits=splits,
                                    alibi_slopes=sl)
    torch.cuda.synchronize()
    rep = Hq // Hkv
    k_rep = np.repeat(workloads.to_f64_numpy(k), rep, axis=1)
    v_rep = np.repeat(workloads.to_f64_numpy(v), rep, axis=1)
    o_ref, lse_ref = oracle.forward(workloads.to_f64_numpy(q), k_rep, v_rep, scale, causal,
                                    alibi_slopes=None if sl is None else sl.double().numpy())
    eo, _ = check_o(f64(o), o_ref, dt)
    el = check_lse(f64(lse), lse_ref)
    log(f"  max|dO|={eo:.2e} max|dlse|={el:.2e}")
