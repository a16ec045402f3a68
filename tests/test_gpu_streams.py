"""The convenience calls with an explicit ``stream=`` argument (runs on the GPU).

Their outputs and temporaries (backward workspace, KV-cache workspace,
ALiBi slopes) must be allocated on the stream the kernels run on.  The
kernels are enqueued on a side stream behind a long-running product, while
the current stream allocates and fills memory of the same sizes over and
over: a temporary allocated on the current stream and freed on return would
be handed to those fills while the side-stream kernels still read it.  Every
result must still match the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import check_grad, check_lse, check_o, f64, log, require_gpu

pytestmark = pytest.mark.gpu


def _churn(nbytes: int, device):
    """Allocate and fill blocks of about nbytes on the current stream, several times."""
    for _ in range(6):
        t = torch.full((nbytes,), 0x7F, dtype=torch.uint8, device=device)
        t.fill_(0xFF)
        del t


def test_convenience_calls_on_explicit_stream():
    ea = require_gpu()
    w = workloads.Workload("stream_arg", 1, 3, 320, 64, "bf16", True, True, seed=44001)
    log(f"explicit stream= {w}")
    x = workloads.make_inputs(w)
    q, k, v, do = (x[n].cuda() for n in ("q", "k", "v", "do"))
    slopes = [0.5, 0.25, 0.125]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    ws_bytes = ea.attn_bwd_workspace_bytes(1, 3, 320, 64)
    with torch.cuda.stream(side):
        a = torch.randn(4096, 4096, device="cuda")
        for _ in range(8):
            a = a @ a * 1e-3            # keeps the side stream busy while the current stream churns
    o, lse = ea.forward(q, k, v, scale=w.scale, causal=True, stream=side)
    g = ea.backward(q, k, v, o, lse, do, scale=w.scale, causal=True, stream=side)
    oa, la = ea.forward_alibi(q, k, v, slopes, scale=w.scale, causal=True, stream=side)
    ga = ea.backward_alibi(q, k, v, oa, la, do, slopes, scale=w.scale, causal=True, stream=side)
    od, ld = ea.forward_dropout(q, k, v, 0.25, 17, 0, scale=w.scale, causal=True, stream=side)
    gd = ea.backward_dropout(q, k, v, od, ld, do, 0.25, 17, 0, scale=w.scale, causal=True, stream=side)
    ok, lk = ea.forward_kvcache(q[:, :, -5:].contiguous(), k, v, scale=w.scale, causal=True, num_splits=4,
                                stream=side)
    _churn(ws_bytes, q.device)
    side.synchronize()
    torch.cuda.synchronize()
    args = [workloads.to_f64_numpy(x[n]) for n in ("q", "k", "v")]
    dov = workloads.to_f64_numpy(x["do"])
    o_ref, l_ref = oracle.forward(*args, w.scale, True)
    check_o(f64(o), o_ref, "bf16")
    check_lse(f64(lse), l_ref)
    for name, t, r in zip(("dQ", "dK", "dV"), g, oracle.backward(*args, dov, w.scale, True)):
        check_grad(f64(t), r, name)
    sl = np.array(slopes)
    o_ref, l_ref = oracle.forward(*args, w.scale, True, alibi_slopes=sl)
    check_o(f64(oa), o_ref, "bf16", "O alibi")
    check_lse(f64(la), l_ref, "lse alibi")
    for name, t, r in zip(("dQ", "dK", "dV"), ga, oracle.backward(*args, dov, w.scale, True, alibi_slopes=sl)):
        check_grad(f64(t), r, name + " alibi")
    o_ref, l_ref = oracle.forward(*args, w.scale, True, dropout=(0.25, 17, 0))
    check_o(f64(od), o_ref, "bf16", "O dropout", gain=4 / 3)
    check_lse(f64(ld), l_ref, "lse dropout")
    for name, t, r in zip(("dQ", "dK", "dV"), gd, oracle.backward(*args, dov, w.scale, True, dropout=(0.25, 17, 0))):
        check_grad(f64(t), r, name + " dropout")
    o_ref, l_ref = oracle.forward(args[0][:, :, -5:], args[1], args[2], w.scale, True)
    check_o(f64(ok), o_ref, "bf16", "O kvcache")
    check_lse(f64(lk), l_ref, "lse kvcache")
