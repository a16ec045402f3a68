"""fp64 CPU oracle for exact scaled-dot-product attention, forward and backward.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
run this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library; the two meet only through the seeded inputs of ``workloads.py``.

Everything is numpy float64 on the already-rounded bf16/fp16 inputs.  The
method is exact (the tiled, online-softmax computation reaches the same
result as plain attention, only in a different order), so the oracle is the
plain definition, written out per (batch, head):

* scores ``S = scale * Q K^T``, with ``S_ij = -inf`` for ``j > i`` when causal
  [page "FlashAttention技术解析 如何让GPT训练速度提升5-9倍", §2.1, the
  ``standard_attention`` sketch (scale 1/sqrt(d_k)); page "Flash Attention V2
  大模型时代的算力救星", §4.2, the ``softmax_scale`` and ``causal`` arguments];
* a row softmax, taken in two passes (row max, then exponentials and their
  sum) [page "突破单卡显存极限：FlashAttention-2技术解析与实战指南", §1];
* ``O = P V`` and, as the one kept per-row statistic, ``lse = m + ln l`` in
  natural log [page "Flash Attention V2 大模型时代的算力救星", §3.2: only the
  softmax normalisation statistics survive the forward pass];
* the backward pass is the exact chain rule of that forward definition,
  with the probabilities recomputed from Q and K [same page, §3.2; page
  "突破单卡显存极限…", §2.2]:
  ``dV = P^T dO``, ``dP = dO V^T``, ``D_i = sum_j P_ij dP_ij``,
  ``dS = P o (dP - D)``, ``dQ = scale dS K``, ``dK = scale dS^T Q``.

``online_softmax_forward_head`` follows the blockwise recurrence of page
"突破单卡显存极限…" §2.1 step by step (running max ``m``, running denominator
``l``, both rescaled by ``exp(m_old - m_new)`` at every block).  It is not used
to check the GPU; it exists so that the tests can pin the recurrence to the
plain definition.

Readings where the pages are silent: the causal mask is top-left aligned
with the diagonal kept; lse is in natural log; dropout is off unless asked
for (its generator and mask layout: ``oracle/philox.py``); the backward pass
differentiates O only (lse receives no gradient).

Optional linear position bias (ALiBi) [page "FlashAttention技术解析 如何让GPT
训练速度提升5-9倍", §4.1 names ALiBi with long contexts; the pages give no
formula]: reading, the published form, a per-head slope ``m_h`` and
``S_ij += -m_h * |(i + Nk - Nq) - j|`` added to the scaled scores before the
softmax; for causal rows this is ``-m_h * (i' - j)`` with ``i'`` the query's
position, non-causal rows take the distance both ways.  The bias is a
constant of the inputs, so the backward formulas are unchanged given P.

Query and key counts may differ (``Nq`` rows of Q against ``Nk`` rows of K and
V), the shape of decoding against a KV cache [page "FlashAttention技术解析
如何让GPT训练速度提升5-9倍", §4.1: the keys and values of earlier positions
are kept and reused].  The pages give no mask for that case; the reading
here is that the ``Nq`` queries are the last ``Nq`` positions of the
sequence whose ``Nk`` keys are cached, so causal query ``i`` sees keys
``j <= i + (Nk - Nq)`` (bottom-right alignment).  With ``Nq == Nk`` this is
the top-left mask above.  Causal with ``Nk < Nq`` leaves rows with no
visible key and is not defined.
"""
from __future__ import annotations

import math
from typing import Iterable, Optional, Tuple

import numpy as np

from . import philox

__all__ = [
    "masked_scores",
    "row_softmax",
    "forward_head",
    "forward_head_rows",
    "backward_head",
    "backward_head_rows",
    "forward",
    "backward",
    "online_softmax_forward_head",
]


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def masked_scores(q, k, scale: float, causal: bool, rows: Optional[np.ndarray] = None,
                  alibi_slope: Optional[float] = None, nk_total: Optional[int] = None) -> np.ndarray:
    """S = scale * Q K^T for the given query rows (all rows by default).

    Causal reading: query i sees keys j <= i + (Nk - Nq), i.e. j <= i
    (top-left, diagonal kept) when Q and K have the same number of rows, and
    the queries are the last Nq positions otherwise; every other entry is -inf.
    ``k`` may hold only the first keys of a longer sequence of ``nk_total``
    keys (positions are those of the whole sequence).
    """
    q = _f64(q)
    k = _f64(k)
    n = q.shape[0]
    nk = k.shape[0] if nk_total is None else int(nk_total)
    if rows is None:
        rows = np.arange(n)
    rows = np.asarray(rows, dtype=np.int64)
    s = float(scale) * (q[rows] @ k.T)
    cols = np.arange(k.shape[0])
    pos = rows[:, None] + (nk - n)       # the queries' positions in the key sequence
    if alibi_slope is not None:
        s = s - float(alibi_slope) * np.abs(pos - cols[None, :])
    if causal:
        s[cols[None, :] > pos] = -np.inf
    return s


def row_softmax(s: np.ndarray) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Two-pass row softmax: returns (P, m, l) with m the row max and l = sum exp(S - m)."""
    m = s.max(axis=1)
    e = np.exp(s - m[:, None])
    l = e.sum(axis=1)
    return e / l[:, None], m, l


def dropout_factor(rows, nq: int, nk: int, dropout) -> Optional[np.ndarray]:
    """The factor Z * 256 / (256 - t) (0 where dropped) for the listed query rows of one head,
    or None without dropout; ``dropout`` is ``(p, seed, offset, bh)``."""
    if dropout is None:
        return None
    p, seed, offset, bh = dropout
    z = philox.keep_mask(bh, nq, nk, p, seed, offset)[np.asarray(rows, dtype=np.int64)]
    return z * philox.keep_scale(p)


def visible_keys(rows, nq: int, nk: int, causal: bool) -> int:
    """Number of leading keys any of the listed query rows may see.

    Causal query i sees keys j <= i + (nk - nq), so keys past the largest such
    bound carry weight exp(-inf) = 0 in every listed row and are left out of
    the sums; that changes no value, only the length of zero tails.  Without
    the mask every key is visible."""
    if not causal or len(rows) == 0:
        return nk
    return int(min(nk, max(1, int(np.max(rows)) + (nk - nq) + 1)))


def forward_head_rows(q, k, v, scale: float, causal: bool, rows, alibi_slope=None,
                      dropout=None) -> Tuple[np.ndarray, np.ndarray]:
    """O and lse of the listed query rows of one head (each row is independent).

    With dropout the probabilities are multiplied by the keep factor before
    the product with V; lse stays that of the softmax itself."""
    nq, nk = np.shape(q)[0], np.shape(k)[0]
    rows = np.asarray(rows, dtype=np.int64)
    kv = visible_keys(rows, nq, nk, causal)
    s = masked_scores(q, _f64(k)[:kv], scale, causal, rows, alibi_slope, nk_total=nk)
    p, m, l = row_softmax(s)
    zf = dropout_factor(rows, nq, nk, dropout)
    o = (p if zf is None else p * zf[:, :kv]) @ _f64(v)[:kv]
    lse = m + np.log(l)
    return o, lse


def forward_head(q, k, v, scale: float, causal: bool, row_block: Optional[int] = None, alibi_slope=None,
                 dropout=None):
    """O [N,d] and lse [N] of one head.

    ``row_block`` only bounds memory for long sequences: the definition is
    evaluated for ``row_block`` query rows at a time (rows never interact).
    """
    n = np.shape(q)[0]
    if row_block is None or row_block >= n:
        return forward_head_rows(q, k, v, scale, causal, np.arange(n), alibi_slope, dropout)
    o = np.empty((n, np.shape(v)[1]))
    lse = np.empty(n)
    for r0 in range(0, n, row_block):
        rows = np.arange(r0, min(n, r0 + row_block))
        o[rows], lse[rows] = forward_head_rows(q, k, v, scale, causal, rows, alibi_slope, dropout)
    return o, lse


def backward_head_rows(q, k, v, do, scale: float, causal: bool, rows, alibi_slope=None, dropout=None):
    """The listed query rows' share of the backward pass of one head (exact chain rule).

    Returns ``(dq, dk, dv)``: the rows' dQ (``[len(rows), d]``; complete, since
    a row's dQ depends on that row alone) and their contributions to dK and dV
    (``[kv, d]``, keys past ``kv`` get nothing from these rows).  dK and dV are
    sums over the query rows, so the contributions of all rows add up to
    them; with the causal mask only rows ``i >= j`` reach key ``j``, so the
    rows ``j0 .. N-1`` alone give the complete dK and dV of the keys
    ``j >= j0``.

    With dropout (keep factor F = Z * 256 / (256 - t), O = (P o F) V):
    ``dV = (P o F)^T dO``, ``dP = F o (dO V^T)``, and the rest as without;
    ``D_i = sum_j P_ij dP_ij`` still equals ``dO_i . O_i``.
    """
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    do = _f64(do)
    n, nk = q.shape[0], k.shape[0]
    rows = np.asarray(rows, dtype=np.int64)
    kv = visible_keys(rows, n, nk, causal)   # keys past kv have P = 0 in these rows
    s = masked_scores(q, k[:kv], scale, causal, rows, alibi_slope, nk_total=nk)
    p, _, _ = row_softmax(s)
    zf = dropout_factor(rows, n, nk, dropout)
    if zf is not None:
        zf = zf[:, :kv]
    dv = (p if zf is None else p * zf).T @ do[rows]
    dp = do[rows] @ v[:kv].T
    if zf is not None:
        dp = dp * zf
    dsum = (p * dp).sum(axis=1)          # D_i = sum_j P_ij dP_ij
    ds = p * (dp - dsum[:, None])
    dq = float(scale) * (ds @ k[:kv])
    dk = float(scale) * (ds.T @ q[rows])
    return dq, dk, dv


def backward_head(q, k, v, do, scale: float, causal: bool, row_block: Optional[int] = None, alibi_slope=None,
                  dropout=None):
    """dQ, dK, dV [N,d] of one head for upstream gradient dO (exact chain rule):
    the shares of all query rows (``backward_head_rows``) put together.

    ``row_block`` evaluates the same sums ``dV = sum_i P_i^T dO_i`` and
    ``dK = scale * sum_i dS_i^T Q_i`` over groups of query rows, to bound
    memory at long N.
    """
    q = _f64(q)
    k = _f64(k)
    n = q.shape[0]
    rb = n if row_block is None else min(row_block, n)
    dq = np.empty_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros((k.shape[0], np.shape(v)[1]))
    for r0 in range(0, n, rb):
        rows = np.arange(r0, min(n, r0 + rb))
        dq_r, dk_r, dv_r = backward_head_rows(q, k, v, do, scale, causal, rows, alibi_slope, dropout)
        kv = dk_r.shape[0]
        dq[rows] = dq_r
        dk[:kv] += dk_r
        dv[:kv] += dv_r
    return dq, dk, dv


def _heads(x) -> Iterable[Tuple[int, int]]:
    b, h = np.shape(x)[:2]
    for bi in range(b):
        for hi in range(h):
            yield bi, hi


def _head_dropout(dropout, bi: int, hi: int, nh: int):
    return None if dropout is None else (dropout[0], dropout[1], dropout[2], bi * nh + hi)


def forward(q, k, v, scale: float, causal: bool, row_block: Optional[int] = None, alibi_slopes=None,
            dropout=None):
    """O [B,H,Nq,d] and lse [B,H,Nq] over all heads (K, V: [B,H,Nk,d]); alibi_slopes: [H] or None;
    dropout: ``(p, seed, offset)`` or None (head (b, h) draws with index b * H + h)."""
    q = _f64(q)
    b, h, n, d = q.shape
    o = np.empty((b, h, n, np.shape(v)[3]))
    lse = np.empty((b, h, n))
    for bi, hi in _heads(q):
        sl = None if alibi_slopes is None else float(alibi_slopes[hi])
        o[bi, hi], lse[bi, hi] = forward_head(q[bi, hi], k[bi, hi], v[bi, hi], scale, causal, row_block, sl,
                                              _head_dropout(dropout, bi, hi, h))
    return o, lse


def backward(q, k, v, do, scale: float, causal: bool, row_block: Optional[int] = None, alibi_slopes=None,
             dropout=None):
    """dQ, dK, dV [B,H,N,d] over all heads; alibi_slopes: [H] or None; dropout: ``(p, seed, offset)`` or None."""
    q = _f64(q)
    dq = np.empty_like(q)
    dk = np.empty_like(q)
    dv = np.empty((q.shape[0], q.shape[1], q.shape[2], np.shape(v)[3]))
    for bi, hi in _heads(q):
        sl = None if alibi_slopes is None else float(alibi_slopes[hi])
        dq[bi, hi], dk[bi, hi], dv[bi, hi] = backward_head(
            q[bi, hi], k[bi, hi], v[bi, hi], do[bi, hi], scale, causal, row_block, sl,
            _head_dropout(dropout, bi, hi, q.shape[1]))
    return dq, dk, dv


def online_softmax_forward_head(q, k, v, scale: float, causal: bool, block: int):
    """Blockwise online-softmax attention of one head, in the pages' step order.

    Page "突破单卡显存极限：FlashAttention-2技术解析与实战指南" §2.1: start with
    m = -inf and l = 0; for each key block X_j take its row max m_j, its
    exponentials f_j = exp(X_j - m_j) and their sum l_j; merge with
    m_new = max(m, m_j) and l_new = exp(m - m_new) l + exp(m_j - m_new) l_j;
    rescale the block weights by exp(m_j - m_new).  The page leaves out the
    output accumulator; the reading used here is
    acc_new = exp(m - m_new) acc + f_j V_j, then m, l <- m_new, l_new, and
    O = acc / l after the last block.  Blocks of keys a row may not see
    (causal) contribute exp(-inf) = 0.
    """
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    n = q.shape[0]
    nk = k.shape[0]
    dv = v.shape[1]
    m = np.full(n, -np.inf)
    l = np.zeros(n)
    acc = np.zeros((n, dv))
    for c0 in range(0, nk, block):
        cols = np.arange(c0, min(nk, c0 + block))
        x = float(scale) * (q @ k[cols].T)
        if causal:
            x[cols[None, :] > np.arange(n)[:, None] + (nk - n)] = -np.inf
        m_j = x.max(axis=1)
        seen = m_j > -np.inf                      # rows with at least one visible key
        f_j = np.zeros_like(x)
        f_j[seen] = np.exp(x[seen] - m_j[seen, None])
        l_j = f_j.sum(axis=1)
        m_new = np.maximum(m, m_j)
        alpha = np.where(m > -np.inf, np.exp(m - m_new, where=m > -np.inf, out=np.zeros(n)), 0.0)
        beta = np.where(seen, np.exp(m_j - m_new, where=seen, out=np.zeros(n)), 0.0)
        l_new = alpha * l + beta * l_j
        f_j = f_j * beta[:, None]
        acc = alpha[:, None] * acc + f_j @ v[cols]
        m, l = m_new, l_new
    o = acc / l[:, None]
    lse = m + np.log(l)
    return o, lse


def scalar_forward_head(q, k, v, scale: float, causal: bool):
    """Pure-Python scalar forward of one head (math.exp / math.fsum), for tiny inputs."""
    n = len(q)
    d = len(q[0])
    dv = len(v[0])
    o = [[0.0] * dv for _ in range(n)]
    lse = [0.0] * n
    for i in range(n):
        js = [j for j in range(len(k)) if (not causal or j <= i + len(k) - n)]
        s = [float(scale) * math.fsum(float(q[i][c]) * float(k[j][c]) for c in range(d)) for j in js]
        mx = max(s)
        e = [math.exp(x - mx) for x in s]
        tot = math.fsum(e)
        for c in range(dv):
            o[i][c] = math.fsum(e[t] * float(v[j][c]) for t, j in enumerate(js)) / tot
        lse[i] = mx + math.log(tot)
    return np.array(o), np.array(lse)
