"""Forward and KV-cache forward on tensors in other layouts (GPU).

attn_fwd_strided and attn_fwd_kvcache_strided take per-tensor (batch, head,
token) strides with a contiguous head dimension.  Each case runs a layout
the callers of attention use ([B, N, H, d] token-major tensors, a packed
[B, N, 3, H, d] QKV buffer, one K and V shared by every head, a KV cache
allocated for more positions than it holds), checks every element against
the fp64 oracle on contiguous copies, checks that the result is bitwise the
one the contiguous call gives (the same kernels, only the addresses
differ), and checks that no element outside the output view was written.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import check_lse, check_o, f64, log, require_gpu

pytestmark = pytest.mark.gpu


def _inputs(B, H, N, d, dt, seed, Nk=None):
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    Nk = N if Nk is None else Nk
    tdt = {"bf16": torch.bfloat16, "fp16": torch.float16}[dt]
    q = torch.randn((B, H, N, d), generator=g).to(tdt)
    k = torch.randn((B, H, Nk, d), generator=g).to(tdt)
    v = torch.randn((B, H, Nk, d), generator=g).to(tdt)
    return q, k, v


def _oracle(q, k, v, scale, causal):
    return oracle.forward(*(workloads.to_f64_numpy(t.contiguous().cpu()) for t in (q, k, v)), scale, causal)


CASES = [(2, 3, 200, 64, "bf16", True), (1, 4, 256, 128, "fp16", False), (2, 2, 129, 128, "bf16", False),
         (1, 2, 1000, 128, "bf16", True)]


@pytest.mark.parametrize("B,H,N,d,dt,causal", CASES)
def test_forward_token_major_layout(B, H, N, d, dt, causal):
    """q, k, v, o stored [B, N, H, d] (viewed as [B, H, N, d])."""
    ea = require_gpu()
    q, k, v = _inputs(B, H, N, d, dt, 41000 + N + d)
    scale = ea.default_scale(d)
    qs, ks, vs = (t.transpose(1, 2).contiguous().cuda().transpose(1, 2) for t in (q, k, v))
    # output view inside a NaN buffer with one extra head per token
    obuf = torch.full((B, N, H + 1, d), float("nan"), dtype=q.dtype, device="cuda")
    o = obuf[:, :, :H].transpose(1, 2)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    log(f"strided fwd NHD B={B} H={H} N={N} d={d} {dt} causal={causal} strides q={qs.stride()} o={o.stride()}")
    ea.attn_fwd(qs, ks, vs, o, lse, scale, causal)
    oc, lc = ea.forward(q.cuda(), k.cuda(), v.cuda(), scale=scale, causal=causal)
    torch.cuda.synchronize()
    o_ref, lse_ref = _oracle(q, k, v, scale, causal)
    check_o(f64(o), o_ref, dt)
    check_lse(f64(lse), lse_ref)
    assert torch.equal(o, oc) and torch.equal(lse, lc), "strided result differs from the contiguous call"
    assert torch.isnan(obuf[:, :, H]).all(), "wrote outside the output view"


def test_forward_packed_qkv_and_shared_kv_heads():
    ea = require_gpu()
    B, H, N, d = 2, 4, 300, 128
    q, k, v = _inputs(B, H, N, d, "bf16", 42001)
    scale = ea.default_scale(d)
    # packed [B, N, 3, H, d]
    qkv = torch.stack([t.transpose(1, 2) for t in (q, k, v)], dim=2).contiguous().cuda()
    qp, kp, vp = (qkv[:, :, i].transpose(1, 2) for i in range(3))
    log(f"strided fwd packed QKV strides {qp.stride()}")
    o, lse = ea.forward(qp, kp, vp, scale=scale, causal=True)
    torch.cuda.synchronize()
    o_ref, lse_ref = _oracle(q, k, v, scale, True)
    check_o(f64(o), o_ref, "bf16")
    check_lse(f64(lse), lse_ref)
    # one K and V for all heads: head stride 0
    k1, v1 = k[:, :1], v[:, :1]
    ke, ve = k1.cuda().expand(B, H, N, d), v1.cuda().expand(B, H, N, d)
    log(f"strided fwd shared K/V heads strides {ke.stride()}")
    o2, lse2 = ea.forward(q.cuda(), ke, ve, scale=scale, causal=False)
    torch.cuda.synchronize()
    o_ref2, lse_ref2 = _oracle(q, k1.expand(B, H, N, d), v1.expand(B, H, N, d), scale, False)
    check_o(f64(o2), o_ref2, "bf16")
    check_lse(f64(lse2), lse_ref2)


@pytest.mark.parametrize("Nq,Nk,Nmax,splits", [(1, 4000, 4096, 0), (8, 1111, 2048, 0), (40, 300, 320, 3)])
def test_kvcache_token_major_cache(Nq, Nk, Nmax, splits):
    """A [B, Nmax, H, d] cache holding Nk positions, queries [B, Nq, H, d]."""
    ea = require_gpu()
    B, H, d = 2, 4, 128
    q, k, v = _inputs(B, H, Nq, d, "bf16", 43000 + Nk, Nk=Nk)
    scale = ea.default_scale(d)
    kc = torch.full((B, Nmax, H, d), float("nan"), dtype=k.dtype)
    vc = torch.full((B, Nmax, H, d), float("nan"), dtype=v.dtype)
    kc[:, :Nk] = k.transpose(1, 2)
    vc[:, :Nk] = v.transpose(1, 2)
    kc, vc = kc.cuda(), vc.cuda()
    ks, vs = kc[:, :Nk].transpose(1, 2), vc[:, :Nk].transpose(1, 2)
    qs = q.transpose(1, 2).contiguous().cuda().transpose(1, 2)
    log(f"strided kvcache Nq={Nq} Nk={Nk} Nmax={Nmax} splits={splits} k strides {ks.stride()}")
    o, lse = ea.forward_kvcache(qs, ks, vs, scale=scale, causal=True, num_splits=splits)
    oc, lc = ea.forward_kvcache(q.cuda(), k.cuda(), v.cuda(), scale=scale, causal=True, num_splits=splits)
    torch.cuda.synchronize()
    o_ref, lse_ref = _oracle(q, k, v, scale, True)
    check_o(f64(o), o_ref, "bf16")
    check_lse(f64(lse), lse_ref)
    assert torch.equal(o.contiguous(), oc) and torch.equal(lse, lc), "strided result differs from the contiguous call"


def _grads_ref(q, k, v, do, scale, causal):
    return oracle.backward(*(workloads.to_f64_numpy(t.contiguous().cpu()) for t in (q, k, v, do)), scale, causal)


@pytest.mark.parametrize("B,H,N,d,dt,causal", [(2, 3, 256, 64, "bf16", True), (1, 2, 100, 128, "fp16", False),
                                               (1, 4, 640, 128, "bf16", True)])
def test_backward_token_major_layout(B, H, N, d, dt, causal):
    """Forward and backward with all eight tensors stored [B, N, H, d]."""
    ea = require_gpu()
    from parity import check_grad
    q, k, v = _inputs(B, H, N, d, dt, 44000 + N + d)
    g = torch.Generator(device="cpu")
    g.manual_seed(44999 + N)
    do = torch.randn((B, H, N, d), generator=g).to(q.dtype)
    scale = ea.default_scale(d)
    nhd = lambda t: t.transpose(1, 2).contiguous().cuda().transpose(1, 2)
    qs, ks, vs, dos = (nhd(t) for t in (q, k, v, do))
    log(f"strided bwd NHD B={B} H={H} N={N} d={d} {dt} causal={causal}")
    o, lse = ea.forward(qs, ks, vs, scale=scale, causal=causal)
    dq, dk, dv = ea.backward(qs, ks, vs, o, lse, dos, scale=scale, causal=causal)
    assert dq.stride() == qs.stride() and not dq.is_contiguous()
    qc, kc, vc, doc = (t.cuda() for t in (q, k, v, do))
    oc, lc = ea.forward(qc, kc, vc, scale=scale, causal=causal)
    gc = ea.backward(qc, kc, vc, oc, lc, doc, scale=scale, causal=causal)
    torch.cuda.synchronize()
    ref = _grads_ref(q, k, v, do, scale, causal)
    for name, gg, gr, gcc in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref, gc):
        check_grad(f64(gg), gr, name)
        assert torch.equal(gg.contiguous(), gcc), f"{name}: strided result differs from the contiguous call"


def test_backward_packed_qkv_and_packed_gradient():
    """q, k, v views of one [B, N, 3, H, d] buffer; dq, dk, dv written into one packed gradient buffer."""
    ea = require_gpu()
    from parity import check_grad
    B, H, N, d = 2, 4, 200, 128
    q, k, v = _inputs(B, H, N, d, "bf16", 45001)
    g = torch.Generator(device="cpu")
    g.manual_seed(45002)
    do = torch.randn((B, H, N, d), generator=g).to(q.dtype)
    scale = ea.default_scale(d)
    qkv = torch.stack([t.transpose(1, 2) for t in (q, k, v)], dim=2).contiguous().cuda()
    qp, kp, vp = (qkv[:, :, i].transpose(1, 2) for i in range(3))
    dqkv = torch.full_like(qkv, float("nan"))
    dqp, dkp, dvp = (dqkv[:, :, i].transpose(1, 2) for i in range(3))
    o, lse = ea.forward(qp, kp, vp, scale=scale, causal=True)
    dos = do.transpose(1, 2).contiguous().cuda().transpose(1, 2)
    ws = torch.empty(ea.attn_bwd_strided_workspace_bytes(B, H, N, d), dtype=torch.uint8, device="cuda")
    log(f"strided bwd packed QKV and packed dQKV, strides {qp.stride()}")
    ea.attn_bwd(qp, kp, vp, o, dos, lse, dqp, dkp, dvp, scale, True, ws)
    torch.cuda.synchronize()
    assert not torch.isnan(dqkv).any(), "a gradient element was not written"
    ref = _grads_ref(q, k, v, do, scale, True)
    for name, gg, gr in zip(("dQ", "dK", "dV"), (dqp, dkp, dvp), ref):
        check_grad(f64(gg), gr, name)


def test_token_major_headline_size_bitwise_equal_to_contiguous():
    """B=4, H=32, N=4096, d=128 causal bf16 (the headline workload, compared with the oracle over every
    element in test_gpu_fullsize.py) with all eight tensors stored [B, N, H, d]: forward and backward
    must give bitwise the contiguous call's results, and write every gradient element."""
    ea = require_gpu()
    w = workloads.WORKLOADS["causal_b4h32n4096d128"]
    x = workloads.make_inputs(w)
    log(f"strided headline size {w.name}: [B, N, H, d] storage, bitwise against the contiguous call")
    nhd = lambda t: t.transpose(1, 2).contiguous().cuda().transpose(1, 2)
    qs, ks, vs, dos = (nhd(x[n]) for n in ("q", "k", "v", "do"))
    obuf = torch.full((w.B, w.N, w.H, w.d), float("nan"), dtype=qs.dtype, device="cuda")
    o = obuf.transpose(1, 2)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda")
    ea.attn_fwd(qs, ks, vs, o, lse, w.scale, True)
    dq, dk, dv = ea.backward(qs, ks, vs, o, lse, dos, scale=w.scale, causal=True)
    qc, kc, vc, doc = (x[n].cuda() for n in ("q", "k", "v", "do"))
    oc, lc = ea.forward(qc, kc, vc, scale=w.scale, causal=True)
    gc = ea.backward(qc, kc, vc, oc, lc, doc, scale=w.scale, causal=True)
    torch.cuda.synchronize()
    assert not torch.isnan(obuf).any(), "an output element was not written"
    assert torch.equal(o, oc) and torch.equal(lse, lc), "strided forward differs from the contiguous call"
    for name, gg, gcc in zip(("dQ", "dK", "dV"), (dq, dk, dv), gc):
        assert dq.stride() == qs.stride()
        assert torch.equal(gg.contiguous(), gcc), f"{name}: strided result differs from the contiguous call"
