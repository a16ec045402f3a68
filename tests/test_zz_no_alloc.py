"""The KV-cache forward without allocation (runs on the GPU): attn_fwd_kvcache_noalloc
keeps its split partials in the library's static scratch buffer instead of a
caller workspace.  Its output must equal, bit for bit, that of
attn_fwd_kvcache on the same inputs (the same kernels and split plan), and
match the fp64 oracle; two calls in a row, the second smaller, check that
what the first call left in the buffer does not leak into the second.
"""
import pytest
import torch

import oracle
import workloads
from parity import check_lse, check_o, f64, log, require_gpu

pytestmark = pytest.mark.gpu


def _run_both(ea, w, splits):
    x = workloads.make_kv_inputs(w)
    q, k, v = (x[n].cuda() for n in ("q", "k", "v"))
    o1, l1 = ea.forward_kvcache(q, k, v, scale=w.scale, causal=w.causal, num_splits=splits)
    o2 = torch.full_like(q, float("nan"))
    l2 = torch.full((w.B, w.H, w.Nq), float("nan"), device="cuda")
    before = torch.cuda.memory_allocated()
    ea.attn_fwd_kvcache_noalloc(q, k, v, o2, l2, w.scale, w.causal, num_splits=splits)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    return x, (o1, l1), (o2, l2)


def test_noalloc_matches_workspace_entry_point_twice():
    ea = require_gpu()
    big = workloads.KvWorkload("na_big", 4, 32, 8, 4096, 128, "bf16", True, seed=45001)
    small = workloads.KvWorkload("na_small", 2, 3, 1, 777, 64, "fp16", True, seed=45002)
    for w, splits in ((big, 0), (small, 5)):
        need = ea.attn_fwd_kvcache_workspace_bytes(w.B, w.H, w.Nq, w.Nk, w.d, splits)
        log(f"noalloc KV-cache {w} splits={splits} partials {need} bytes")
        assert 0 < need <= ea.ATTN_KV_SCRATCH_BYTES
        x, (o1, l1), (o2, l2) = _run_both(ea, w, splits)
        assert torch.equal(o1, o2) and torch.equal(l1, l2)
        o_ref, l_ref = oracle.forward(*(workloads.to_f64_numpy(x[n]) for n in ("q", "k", "v")), w.scale, w.causal)
        check_o(f64(o2), o_ref, w.dtype)
        check_lse(f64(l2), l_ref)


def test_noalloc_rejects_calls_beyond_the_scratch_buffer():
    ea = require_gpu()
    B, H, Nq, Nk, d = 8, 64, 64, 8192, 128
    need = ea.attn_fwd_kvcache_workspace_bytes(B, H, Nq, Nk, d, 64)
    assert need > ea.ATTN_KV_SCRATCH_BYTES
    q = torch.zeros((B, H, Nq, d), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((B, H, Nk, d), dtype=torch.bfloat16, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Nq), device="cuda")
    with pytest.raises(ea.AttnError) as exc:
        ea.attn_fwd_kvcache_noalloc(q, k, k, o, lse, 0.125, True, num_splits=64)
    assert exc.value.status == 13
