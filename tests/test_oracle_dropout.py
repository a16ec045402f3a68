"""Pins of the oracle's dropout: the generator, the mask layout and the gradients.

* Philox4x32-10 reproduces its authors' published known-answer vectors
  (tests/golden/philox4x32_10_kat.txt);
* the mask assembled for a whole head equals, element by element, the byte
  the stated layout names in a single generator call;
* the drop rate and the independence of neighbouring rows and keys match a
  Bernoulli(t / 256) draw within binomial bounds;
* p = 0 reduces to attention without dropout, bit for bit;
* the expected output over seeds is the output without dropout (the keep
  factor has mean 1);
* central finite differences of L = sum(O * dO) with a fixed mask agree with
  the backward, and D_i = dO_i . O_i still holds;
* planted mistakes (dP not masked, V masked twice, the wrong scale) fail
  the finite-difference check.
"""
import os

import numpy as np
import pytest

import oracle
from oracle import attention as A
from oracle import philox

KAT = os.path.join(os.path.dirname(__file__), "golden", "philox4x32_10_kat.txt")


def test_philox_known_answers():
    rows = [ln.split() for ln in open(KAT) if ln.strip() and not ln.startswith("#")]
    assert len(rows) == 3
    for r in rows:
        w = [int(x, 16) for x in r]
        out = philox.philox4x32_10(np.array(w[:4], dtype=np.uint64), (w[4], w[5]))
        assert [int(x) for x in out] == w[6:]


def test_mask_layout_element_by_element():
    seed, off, bh = 0x1234_5678_9ABC_DEF0, 7, 5
    nq, nk = 11, 14
    d = philox.draws(bh, nq, nk, seed, off)
    for i in range(nq):
        for j in range(nk):
            out = philox.philox4x32_10(np.array([i // 4, j // 4, bh, off], dtype=np.uint64),
                                       (seed & 0xFFFFFFFF, seed >> 32))
            assert d[i, j] == (int(out[i % 4]) >> (8 * (j % 4))) & 0xFF, (i, j)


def test_threshold_and_scale():
    assert philox.dropout_threshold(0.0) == 0 and philox.keep_scale(0.0) == 1.0
    assert philox.dropout_threshold(0.1) == 26 and philox.keep_scale(0.1) == 256 / 230
    assert philox.dropout_threshold(0.5) == 128 and philox.keep_scale(0.5) == 2.0
    assert philox.dropout_threshold(255 / 256) == 255 and philox.keep_scale(255 / 256) == 256.0
    assert philox.dropout_threshold(1 / 512) == 1
    for bad in (1.0, -0.1, float("nan"), 0.001, 1 / 512 - 1e-9, 511 / 512, 0.999):
        with pytest.raises(ValueError):
            philox.dropout_threshold(bad)


@pytest.mark.parametrize("p", [0.1, 0.5])
def test_drop_rate_and_independence(p):
    t = philox.dropout_threshold(p)
    q = t / 256
    z = philox.keep_mask(3, 512, 512, p, seed=99, offset=0)
    n = z.size
    dropped = 1.0 - z.mean()
    assert abs(dropped - q) <= 5 * np.sqrt(q * (1 - q) / n)
    # neighbouring rows / keys (same and different generator calls) agree as independent draws would
    same = q * q + (1 - q) * (1 - q)
    for a, b in ((z[:-1], z[1:]), (z[:, :-1], z[:, 1:]), (z[:-4], z[4:]), (z[:, :-4], z[:, 4:])):
        agree = (a == b).mean()
        assert abs(agree - same) <= 5 * np.sqrt(same * (1 - same) / a.size)
    # heads, seeds and offsets give different masks
    assert (z != philox.keep_mask(4, 512, 512, p, 99, 0)).any()
    assert (z != philox.keep_mask(3, 512, 512, p, 100, 0)).any()
    assert (z != philox.keep_mask(3, 512, 512, p, 99, 1)).any()


def _rand(rng, b, h, n, d):
    return [rng.standard_normal((b, h, n, d)) for _ in range(4)]


@pytest.mark.parametrize("causal", [False, True])
def test_p_zero_is_plain_attention(causal):
    rng = np.random.default_rng(5)
    q, k, v, do = _rand(rng, 2, 2, 13, 8)
    o0, l0 = oracle.forward(q, k, v, 0.4, causal)
    o1, l1 = oracle.forward(q, k, v, 0.4, causal, dropout=(0.0, 77, 3))
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)
    g0 = oracle.backward(q, k, v, do, 0.4, causal)
    g1 = oracle.backward(q, k, v, do, 0.4, causal, dropout=(0.0, 77, 3))
    for a, b in zip(g0, g1):
        assert np.array_equal(a, b)


def test_expectation_over_seeds_is_plain_attention():
    rng = np.random.default_rng(6)
    q, k, v, _ = _rand(rng, 1, 1, 9, 4)
    o0, l0 = oracle.forward(q, k, v, 0.5, True)
    n = 3000
    acc = np.zeros_like(o0)
    sq = np.zeros_like(o0)
    for s in range(n):
        o, lse = oracle.forward(q, k, v, 0.5, True, dropout=(0.25, s, 0))
        assert np.array_equal(lse, l0)          # lse is that of the softmax itself
        acc += o
        sq += o * o
    mean = acc / n
    sd = np.sqrt(np.maximum(sq / n - mean * mean, 0) / n)
    assert (np.abs(mean - o0) <= 5 * sd + 1e-12).all()


def _fd_check(fwd, bwd, causal, nq, nk, seed):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((nq, 3))
    k = rng.standard_normal((nk, 3))
    v = rng.standard_normal((nk, 2))
    do = rng.standard_normal((nq, 2))
    h = 1e-6
    grads = bwd(q, k, v, do)
    worst = 0.0
    for which, g in enumerate(grads):
        base = [q, k, v]
        fd = np.zeros_like(g)
        for idx in np.ndindex(*g.shape):
            plus = [x.copy() for x in base]
            minus = [x.copy() for x in base]
            plus[which][idx] += h
            minus[which][idx] -= h
            fd[idx] = ((fwd(*plus) * do).sum() - (fwd(*minus) * do).sum()) / (2 * h)
        worst = max(worst, np.linalg.norm(fd - g) / max(np.linalg.norm(fd), 1e-12))
    return worst


DROP = (0.3, 1234, 2, 1)      # p, seed, offset, bh


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("nq,nk", [(6, 6), (5, 9), (9, 9)])
def test_dropout_finite_differences(causal, nq, nk):
    fwd = lambda q, k, v: A.forward_head(q, k, v, 0.7, causal, dropout=DROP)[0]
    bwd = lambda q, k, v, do: A.backward_head(q, k, v, do, 0.7, causal, dropout=DROP)
    z = philox.keep_mask(1, nq, nk, 0.3, 1234, 2)
    assert 0 < z.mean() < 1                     # some dropped, some kept
    assert _fd_check(fwd, bwd, causal, nq, nk, 40 + nq + nk) <= 1e-6


def test_delta_identity_with_dropout():
    rng = np.random.default_rng(8)
    q, k, v, do = (x[0, 0] for x in _rand(rng, 1, 1, 10, 4))
    o, _ = A.forward_head(q, k, v, 0.6, True, dropout=DROP)
    s = A.masked_scores(q, k, 0.6, True)
    p, _, _ = A.row_softmax(s)
    f = A.dropout_factor(np.arange(10), 10, 10, DROP)
    dp = (do @ v.T) * f
    assert np.allclose((p * dp).sum(1), (do * o).sum(1), rtol=1e-12, atol=1e-12)


def _planted_bwd(kind):
    def bwd(q, k, v, do):
        s = A.masked_scores(q, k, 0.7, False)
        p, _, _ = A.row_softmax(s)
        f = A.dropout_factor(np.arange(q.shape[0]), q.shape[0], k.shape[0], DROP)
        dv = (p * f).T @ do
        dp = do @ v.T
        if kind == "dP not masked":
            pass
        elif kind == "V side masked twice":
            dv = (p * f * f).T @ do
            dp = dp * f
        elif kind == "mask without scale":
            dp = dp * (f > 0)
        ds = p * (dp - (p * dp).sum(1, keepdims=True))
        return 0.7 * ds @ k, 0.7 * ds.T @ q, dv
    return bwd


@pytest.mark.parametrize("kind", ["dP not masked", "V side masked twice", "mask without scale"])
def test_planted_dropout_mistake_is_caught(kind):
    fwd = lambda q, k, v: A.forward_head(q, k, v, 0.7, False, dropout=DROP)[0]
    assert _fd_check(fwd, _planted_bwd(kind), False, 6, 7, 3) > 1e-3


def _pin_head_index(fwd, bwd):
    """Head (b, h) of a [B, H, ...] call draws its mask with generator index
    b * H + h.  With V (and dO) the identity, O[i, j] = P_ij F_ij and
    dV[j, i] = P_ij F_ij, so the zeros of O and of dV^T are exactly the
    dropped positions; every head's pattern is compared with the generator's
    draws at that index.  Non-causal with distinct scores, so P_ij > 0."""
    B, H, n = 2, 3, 12
    p, seed, off = 0.5, 0x1F2E3D4C5B6A7988, 11
    t = philox.dropout_threshold(p)
    rng = np.random.default_rng(21)
    q = rng.standard_normal((B, H, n, 4))
    k = rng.standard_normal((B, H, n, 4))
    eye = np.broadcast_to(np.eye(n), (B, H, n, n)).copy()
    o, _ = fwd(q, k, eye, 0.5, False, dropout=(p, seed, off))
    _, _, dv = bwd(q, k, eye, eye, 0.5, False, dropout=(p, seed, off))
    for b in range(B):
        for h in range(H):
            dropped = philox.draws(b * H + h, n, n, seed, off) < t
            assert 0 < dropped.mean() < 1
            assert np.array_equal(o[b, h] == 0.0, dropped), (b, h)
            assert np.array_equal(dv[b, h].T == 0.0, dropped), (b, h)


def test_multihead_dropout_uses_head_index_b_times_H_plus_h():
    _pin_head_index(oracle.forward, oracle.backward)


@pytest.mark.parametrize("index", ["h*B+b", "h", "b"])
def test_planted_head_index_mistake_is_caught(index, monkeypatch):
    """A wrapper that numbers heads any other way fails the pin above."""
    def wrong(dropout, bi, hi, nh):
        if dropout is None:
            return None
        nb = 2   # the pin's batch size
        idx = {"h*B+b": hi * nb + bi, "h": hi, "b": bi}[index]
        return (dropout[0], dropout[1], dropout[2], idx)
    monkeypatch.setattr(A, "_head_dropout", wrong)
    with pytest.raises(AssertionError):
        _pin_head_index(A.forward, A.backward)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("nq,nk", [(13, 13), (9, 29)])
@pytest.mark.parametrize("drop", [None, (0.3, 5, 1, 2)])
def test_row_blocks_equal_unblocked_kv_shapes_and_dropout(causal, nq, nk, drop):
    """Evaluating rows in blocks (which leaves out keys no row of a causal
    block may see) gives the values of the unblocked evaluation."""
    rng = np.random.default_rng(31 + nq + nk)
    q = rng.standard_normal((nq, 5))
    k = rng.standard_normal((nk, 5))
    v = rng.standard_normal((nk, 3))
    do = rng.standard_normal((nq, 3))
    o1, l1 = A.forward_head(q, k, v, 0.6, causal, dropout=drop)
    o2, l2 = A.forward_head(q, k, v, 0.6, causal, row_block=4, dropout=drop)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-13)
    g1 = A.backward_head(q, k, v, do, 0.6, causal, dropout=drop)
    g2 = A.backward_head(q, k, v, do, 0.6, causal, row_block=4, dropout=drop)
    for a, b in zip(g1, g2):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)
