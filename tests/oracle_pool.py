"""Whole-tensor comparison of GPU results with the fp64 oracle at full workload size.

The oracle evaluates one (batch, head) at a time, so the heads are spread
over a pool of worker processes (one BLAS thread each).  Each worker computes
its head's oracle result and compares it with the GPU result right there,
returning only error sums and maxima; the parent adds them up into the
metrics over the whole tensors:

* O: max|err| and mean|err| over all B*H*N*d elements, the count of
  elements over their bound (1e-2, or half an output ulp + 1e-3 where
  |O_ref| >= 4: the output format's own rounding exceeds 1e-2 there), the
  count of such |O_ref| >= 4 elements, and the rounding floor of the oracle
  itself, max|round(O_ref) - O_ref|;
* lse: max|err| over all B*H*N rows;
* dQ, dK, dV: ||G - G_ref||_F / ||G_ref||_F over each whole tensor, plus the
  worst single head as a diagnostic.

This module imports numpy and the oracle only (workers start with the spawn
method and never load torch or the HIP library).
"""
from __future__ import annotations

import multiprocessing as mp
import os
from typing import Dict, Iterator, Optional, Tuple

import numpy as np

_MANT = {"bf16": 7, "fp16": 10}


def default_workers() -> int:
    """Worker processes: the host's CPU count, at most 16."""
    env = os.environ.get("ATTN_ORACLE_WORKERS")
    if env:
        return max(1, int(env))
    return max(1, min(16, os.cpu_count() or 1))


def half_ulp(x: np.ndarray, dtype: str) -> np.ndarray:
    e = np.floor(np.log2(np.maximum(np.abs(x), 1e-30)))
    return 0.5 * np.exp2(e - _MANT[dtype])


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round fp64 values to the 16-bit format (nearest even, via fp32) and back."""
    if dtype == "fp16":
        return x.astype(np.float16).astype(np.float64)
    f = x.astype(np.float32).view(np.uint32).astype(np.uint64)
    f = (f + 0x7FFF + ((f >> 16) & 1)) & 0xFFFF0000
    return f.astype(np.uint32).view(np.float32).astype(np.float64)


def _head_task(task):
    """Oracle of one head and its comparison with the GPU result (in a worker)."""
    from oracle import attention as A

    (b, h, scale, causal, dtype, row_block, q, k, v, do, o_gpu, lse_gpu, grads, dropout, gain, slope) = task
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    out = {"b": b, "h": h}
    if o_gpu is not None:
        o_ref, lse_ref = A.forward_head(q, k, v, scale, causal, row_block=row_block, alibi_slope=slope,
                                        dropout=dropout)
        err = np.abs(o_gpu.astype(np.float64) - o_ref)
        big = np.abs(o_ref) >= 4.0
        bound = np.where(big, half_ulp(o_ref, dtype) + 1e-3 * gain, 1e-2 * gain)
        over = err > bound
        out["o_max"] = float(err.max())
        out["o_sum"] = float(err.sum())
        out["o_n"] = int(err.size)
        out["o_over"] = int(over.sum())
        out["o_big"] = int(big.sum())
        out["o_floor"] = float(np.abs(round_to(o_ref, dtype) - o_ref).max())
        out["o_half_ulp_sum"] = float(half_ulp(o_ref, dtype).sum())
        out["o_err_sq"] = float(np.sum(err ** 2))
        out["o_ref_sq"] = float(np.sum(o_ref ** 2))
        if out["o_over"]:
            i = np.unravel_index(int(np.argmax(np.where(over, err - bound, -np.inf))), err.shape)
            out["o_worst_over"] = (int(i[0]), int(i[1]), float(o_gpu[i]), float(o_ref[i]))
        out["lse_max"] = float(np.abs(lse_gpu.astype(np.float64) - lse_ref).max())
        out["finite"] = bool(np.isfinite(o_gpu).all() and np.isfinite(lse_gpu).all())
    if grads is not None:
        ref = A.backward_head(q, k, v, np.asarray(do, dtype=np.float64), scale, causal, row_block=row_block,
                              alibi_slope=slope, dropout=dropout)
        for name, g, gr in zip(("dq", "dk", "dv"), grads, ref):
            g = g.astype(np.float64)
            out[name + "_num"] = float(np.sum((g - gr) ** 2))
            out[name + "_den"] = float(np.sum(gr ** 2))
            out[name + "_finite"] = bool(np.isfinite(g).all())
    return out


def _f32(t) -> np.ndarray:
    """A CPU torch tensor (any float dtype) as an fp32 numpy array (exact for 16-bit values)."""
    return t.float().numpy() if hasattr(t, "float") else np.asarray(t, dtype=np.float32)


def compare_full(w, x, o=None, lse=None, grads=None, workers: Optional[int] = None,
                 row_block: int = 512, dropout=None, alibi_slopes=None) -> Dict[str, float]:
    """Compare GPU outputs of workload ``w`` (inputs ``x``: CPU tensors of the I/O dtype) with the oracle
    over every head.  ``o``, ``lse``: the forward outputs (CPU tensors) or None; ``grads``: (dq, dk, dv)
    CPU tensors or None; ``dropout``: ``(p, seed, offset)`` or None (head (b, h) draws with index
    b * H + h); ``alibi_slopes``: the H per-head slopes of a linear position bias, or None.  With dropout the O bounds other than the output rounding floor grow by the keep factor
    k = 256 / (256 - t) (every rounding made before the final multiplication by k is multiplied by it).
    Returns the whole-tensor metrics (see the module docstring)."""
    from oracle import philox

    workers = workers or default_workers()
    gain = 1.0 if dropout is None else philox.keep_scale(dropout[0])

    def tasks() -> Iterator[Tuple]:
        for b in range(w.B):
            for h in range(w.H):
                yield (b, h, float(w.scale), bool(w.causal), w.dtype, row_block,
                       _f32(x["q"][b, h]), _f32(x["k"][b, h]), _f32(x["v"][b, h]),
                       None if grads is None else _f32(x["do"][b, h]),
                       None if o is None else _f32(o[b, h]), None if lse is None else lse[b, h].numpy(),
                       None if grads is None else tuple(_f32(g[b, h]) for g in grads),
                       None if dropout is None else (dropout[0], dropout[1], dropout[2], b * w.H + h), gain,
                       None if alibi_slopes is None else float(alibi_slopes[h]))

    saved = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")}
    for k in saved:
        os.environ[k] = "1"
    try:
        ctx = mp.get_context("spawn")
        with ctx.Pool(workers) as pool:
            results = list(pool.imap_unordered(_head_task, tasks()))
    finally:
        for k, val in saved.items():
            if val is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = val

    m: Dict[str, float] = {"heads": len(results), "workers": workers}
    if o is not None:
        n = sum(r["o_n"] for r in results)
        m["o_max"] = max(r["o_max"] for r in results)
        m["o_mean"] = sum(r["o_sum"] for r in results) / n
        m["o_elements"] = n
        m["o_over"] = sum(r["o_over"] for r in results)
        m["o_big"] = sum(r["o_big"] for r in results)
        m["o_floor"] = max(r["o_floor"] for r in results)
        m["o_mean_half_ulp"] = sum(r["o_half_ulp_sum"] for r in results) / n
        m["o_rel_fro"] = float(np.sqrt(sum(r["o_err_sq"] for r in results) / sum(r["o_ref_sq"] for r in results)))
        m["lse_max"] = max(r["lse_max"] for r in results)
        m["finite"] = all(r["finite"] for r in results)
        over = [r for r in results if r.get("o_worst_over")]
        if over:
            r = over[0]
            m["o_worst_over"] = (r["b"], r["h"]) + r["o_worst_over"]
    if grads is not None:
        for name in ("dq", "dk", "dv"):
            num = sum(r[name + "_num"] for r in results)
            den = sum(r[name + "_den"] for r in results)
            m[name + "_rel_fro"] = float(np.sqrt(num / den)) if den > 0 else float(np.sqrt(num))
            m[name + "_worst_head"] = max(float(np.sqrt(r[name + "_num"] / r[name + "_den"])) if r[name + "_den"] > 0
                                          else float(np.sqrt(r[name + "_num"])) for r in results)
            m[name + "_finite"] = all(r[name + "_finite"] for r in results)
    return m
