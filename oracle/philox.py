"""Philox4x32-10 counter-based generator, and the dropout keep-mask drawn from it.

TEST INFRASTRUCTURE ONLY (see the package docstring): the HIP library has
its own implementation of the same published generator; the two share no code.

Generator: Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as easy
as 1, 2, 3" (SC 2011), the Philox-4x32 bijection with 10 rounds.  A 128-bit
counter (four 32-bit words c0..c3) and a 64-bit key (k0, k1) map to four
32-bit words.  One round multiplies c0 by 0xD2511F53 and c2 by 0xCD9E8D57
as 32 x 32 -> 64-bit products and sets
    (c0, c1, c2, c3) <- (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2), hi(M0 c0) ^ c3 ^ k1, lo(M0 c0));
between rounds the key advances by the Weyl increments (0x9E3779B9, 0xBB67AE85).

Dropout on the attention probabilities [page "FlashAttention技术解析 如何让
GPT训练速度提升5-9倍", §2.2: dropout is one of the elementwise steps fused
into the attention kernel; page "Flash Attention V2 大模型时代的算力救星"
§4.2, the ``dropout_p`` argument].  The pages name no generator and no mask
layout; the reading here:

* the probability ``p`` is taken in steps of 1/256: ``t = floor(256 p + 1/2)``
  (0 <= t <= 255; a positive ``p`` that would give ``t = 0``, or a ``p`` that
  would give ``t = 256``, is rejected), an element is dropped when its 8-bit
  draw is below ``t``,
  and kept elements are scaled by ``256 / (256 - t)``;
* the draws of the 4 x 4 block of (query, key) positions
  ``(4a .. 4a+3, 4b .. 4b+3)`` of head ``bh = b * H + h`` come from one
  generator call, counter ``(a, b, bh, offset)``, key ``(seed mod 2^32,
  seed div 2^32)``; query ``4a + u`` takes output word ``u`` and key
  ``4b + c`` takes byte ``c`` of that word (byte 0 the least significant).

Query and key indices are row indices of Q and of K (not positions shifted
by ``Nk - Nq``).
"""
from __future__ import annotations

import numpy as np

M0 = np.uint64(0xD2511F53)
M1 = np.uint64(0xCD9E8D57)
W0 = 0x9E3779B9
W1 = 0xBB67AE85
MASK32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(counter, key):
    """Philox4x32-10 on arrays: ``counter`` is a (..., 4) array of uint32 words,
    ``key`` a pair of uint32; returns the (..., 4) uint32 output."""
    c = np.asarray(counter, dtype=np.uint64) & MASK32
    c0, c1, c2, c3 = (c[..., i] for i in range(4))
    k0, k1 = int(key[0]) & 0xFFFFFFFF, int(key[1]) & 0xFFFFFFFF
    for rnd in range(10):
        if rnd:
            k0 = (k0 + W0) & 0xFFFFFFFF
            k1 = (k1 + W1) & 0xFFFFFFFF
        p0 = M0 * c0          # < 2^64: exact in uint64
        p1 = M1 * c2
        c0, c1, c2, c3 = ((p1 >> np.uint64(32)) ^ c1 ^ np.uint64(k0), p1 & MASK32,
                          (p0 >> np.uint64(32)) ^ c3 ^ np.uint64(k1), p0 & MASK32)
    return np.stack([c0, c1, c2, c3], axis=-1).astype(np.uint32)


def dropout_threshold(p: float) -> int:
    """The 8-bit drop threshold t for probability p (elements with draw < t are dropped).

    p is taken to the nearest step of 1/256; a p the 8-bit draws cannot
    realise within half a step (a positive p below 1/512, which would give
    t = 0, or p >= 511/512, which would give t = 256) is rejected."""
    if not (0.0 <= p < 1.0):
        raise ValueError("dropout probability must lie in [0, 1)")
    t = int(np.floor(256.0 * p + 0.5))
    if t > 255 or (t == 0 and p > 0.0):
        raise ValueError("dropout probability must be 0 or lie in [1/512, 511/512)")
    return t


def keep_scale(p: float) -> float:
    """The factor 256 / (256 - t) applied to kept elements."""
    return 256.0 / (256 - dropout_threshold(p))


def draws(bh: int, nq: int, nk: int, seed: int, offset: int) -> np.ndarray:
    """The 8-bit draws of head ``bh`` for queries 0..nq-1 and keys 0..nk-1 (uint8, [nq, nk])."""
    qa = (nq + 3) // 4
    kb = (nk + 3) // 4
    a, b = np.meshgrid(np.arange(qa, dtype=np.uint64), np.arange(kb, dtype=np.uint64), indexing="ij")
    ctr = np.stack([a, b, np.full_like(a, bh), np.full_like(a, offset & 0xFFFFFFFF)], axis=-1)
    out = philox4x32_10(ctr, (seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF))   # [qa, kb, 4] words
    # query 4a+u <- word u; key 4b+c <- byte c
    by = np.stack([(out >> np.uint32(8 * c)) & np.uint32(0xFF) for c in range(4)], axis=-1)   # [qa, kb, u, c]
    full = by.transpose(0, 2, 1, 3).reshape(qa * 4, kb * 4).astype(np.uint8)
    return full[:nq, :nk]


def keep_mask(bh: int, nq: int, nk: int, p: float, seed: int, offset: int) -> np.ndarray:
    """Boolean keep mask of head ``bh`` ([nq, nk]): draw >= t."""
    return draws(bh, nq, nk, seed, offset) >= dropout_threshold(p)
