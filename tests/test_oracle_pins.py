"""Pins of the fp64 oracle to facts it does not compute itself.

Each check compares the oracle with something fixed independently of its
code: hand-derived worked examples (tests/golden), closed forms, invariants of
softmax attention, a pure-Python scalar evaluation, torch's fp64 CPU
``scaled_dot_product_attention`` (a library routine for the textbook
definition) with its autograd, and central finite differences.  The last test
plants plausible mistakes in copies of the oracle's functions and checks that
at least one pin rejects each of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as A

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")


def _ev(x):
    if isinstance(x, (int, float)):
        return float(x)
    return float(eval(x, {"__builtins__": {}}, {"ln": math.log}))  # fixture expressions only


def _arr(x):
    return np.array([[_ev(e) for e in row] for row in x]) if isinstance(x[0], list) else np.array([_ev(e) for e in x])


def _rand(rng, n, d, dv=None):
    dv = d if dv is None else dv
    return rng.standard_normal((n, d)), rng.standard_normal((n, d)), rng.standard_normal((n, dv))


# ---------------------------------------------------------------- the pin suite
# Written against function arguments so that the planted-mistake test can run
# the very same checks on mutated copies of the oracle.

def pin_golden(fwd, bwd):
    with open(GOLDEN) as f:
        ex = json.load(f)["examples"]
    for e in ex:
        q, k, v, do = (_arr(e[n]) for n in ("q", "k", "v", "do"))
        for causal, key in ((False, "noncausal"), (True, "causal")):
            ref = e[key]
            o, lse = fwd(q, k, v, e["scale"], causal)
            np.testing.assert_allclose(o, _arr(ref["o"]), rtol=0, atol=1e-13)
            np.testing.assert_allclose(lse, _arr(ref["lse"]), rtol=0, atol=1e-13)
            dq, dk, dv = bwd(q, k, v, do, e["scale"], causal)
            np.testing.assert_allclose(dq, _arr(ref["dq"]), rtol=0, atol=1e-13)
            np.testing.assert_allclose(dk, _arr(ref["dk"]), rtol=0, atol=1e-13)
            np.testing.assert_allclose(dv, _arr(ref["dv"]), rtol=0, atol=1e-13)


def pin_uniform_scores(fwd, bwd):
    """Q = 0 makes every visible score equal: O_i is the mean of the visible V rows, lse_i = ln(count)."""
    rng = np.random.default_rng(3)
    n, d = 9, 4
    _, k, v = _rand(rng, n, d)
    q = np.zeros((n, d))
    for causal in (False, True):
        o, lse = fwd(q, k, v, 0.7, causal)
        cnt = np.arange(1, n + 1) if causal else np.full(n, n)
        mean = np.cumsum(v, axis=0) / cnt[:, None] if causal else np.broadcast_to(v.mean(0), v.shape)
        np.testing.assert_allclose(o, mean, rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse, np.log(cnt), rtol=0, atol=1e-13)


def pin_one_hot(fwd, bwd):
    """A score that beats all others in its row by >= 60 selects that single V row."""
    rng = np.random.default_rng(4)
    n = 8
    perm = rng.permutation(n)
    q = np.eye(n)[perm] * 70.0            # row i points at key perm[i]
    k = np.eye(n)
    v = rng.standard_normal((n, 3))
    o, lse = fwd(q, k, v, 1.0, False)
    np.testing.assert_allclose(o, v[perm], rtol=0, atol=1e-15)  # off-target weight < e^-70
    np.testing.assert_allclose(lse, np.full(n, 70.0), rtol=0, atol=1e-12)


def pin_first_row_causal(fwd, bwd):
    rng = np.random.default_rng(5)
    q, k, v = _rand(rng, 6, 5)
    o, lse = fwd(q, k, v, 0.3, True)
    np.testing.assert_allclose(o[0], v[0], rtol=0, atol=1e-14)
    assert abs(lse[0] - 0.3 * float(q[0] @ k[0])) < 1e-14


def pin_torch_sdpa(fwd, bwd):
    """torch's fp64 CPU scaled_dot_product_attention and its autograd (library routine)."""
    rng = np.random.default_rng(6)
    for causal in (False, True):
        for n, d in ((7, 3), (16, 8), (33, 16)):
            q, k, v = _rand(rng, n, d)
            do = rng.standard_normal((n, d))
            tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
            to = torch.nn.functional.scaled_dot_product_attention(
                tq[None, None], tk[None, None], tv[None, None], is_causal=causal, scale=0.37)[0, 0]
            to.backward(torch.tensor(do))
            o, _ = fwd(q, k, v, 0.37, causal)
            dq, dk, dv = bwd(q, k, v, do, 0.37, causal)
            np.testing.assert_allclose(o, to.detach().numpy(), rtol=0, atol=1e-12)
            np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=0, atol=1e-12)
            np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=0, atol=1e-12)
            np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=0, atol=1e-12)


def pin_finite_differences(fwd, bwd):
    """Central differences (h = 1e-6) of L = sum(O * dO) on tiny shapes; relative error <= 1e-6."""
    rng = np.random.default_rng(7)
    h = 1e-6
    for causal in (False, True):
        for n in (1, 3, 7):
            for d in (2, 3):
                q, k, v = _rand(rng, n, d)
                do = rng.standard_normal((n, d))
                grads = bwd(q, k, v, do, 0.9, causal)
                for which, g in zip(range(3), grads):
                    base = [q, k, v]
                    fd = np.zeros_like(g)
                    for idx in np.ndindex(*g.shape):
                        plus = [x.copy() for x in base]
                        minus = [x.copy() for x in base]
                        plus[which][idx] += h
                        minus[which][idx] -= h
                        lp = float((fwd(*plus, 0.9, causal)[0] * do).sum())
                        lm = float((fwd(*minus, 0.9, causal)[0] * do).sum())
                        fd[idx] = (lp - lm) / (2 * h)
                    err = np.linalg.norm(fd - g) / max(np.linalg.norm(fd), 1e-300)
                    if np.linalg.norm(fd) < 1e-9:          # e.g. N = 1: gradient of Q and K is 0
                        assert np.abs(g).max() < 1e-8
                    else:
                        assert err <= 1e-6, (causal, n, d, which, err)


def pin_gradient_invariants(fwd, bwd):
    rng = np.random.default_rng(8)
    n, d = 12, 5
    for causal in (False, True):
        q, k, v = _rand(rng, n, d)
        do = rng.standard_normal((n, d))
        dq, dk, dv = bwd(q, k, v, do, 0.6, causal)
        o, _ = fwd(q, k, v, 0.6, causal)
        # every row of dS sums to zero (softmax is shift invariant), so sum_j dK_j = 0
        np.testing.assert_allclose(dk.sum(0), 0.0, atol=1e-12)
        # every row of P sums to one, so sum_j dV_j = sum_i dO_i
        np.testing.assert_allclose(dv.sum(0), do.sum(0), atol=1e-12)
        # all keys equal: scores do not depend on Q, so dQ = 0
        k_same = np.broadcast_to(k[:1], k.shape).copy()
        dq2, _, _ = bwd(q, k_same, v, do, 0.6, causal)
        np.testing.assert_allclose(dq2, 0.0, atol=1e-12)
        # all values equal: O does not depend on the scores, so dQ = dK = 0
        v_same = np.broadcast_to(v[:1], v.shape).copy()
        dq3, dk3, _ = bwd(q, k, v_same, do, 0.6, causal)
        np.testing.assert_allclose(dq3, 0.0, atol=1e-12)
        np.testing.assert_allclose(dk3, 0.0, atol=1e-12)
        # D_i = dO_i . O_i holds for the P that the backward pass recomputes
        s = A.masked_scores(q, k, 0.6, causal)
        p, _, _ = A.row_softmax(s)
        np.testing.assert_allclose((p * (do @ v.T)).sum(1), (do * o).sum(1), atol=1e-12)


PINS = [pin_golden, pin_uniform_scores, pin_one_hot, pin_first_row_causal,
        pin_torch_sdpa, pin_finite_differences, pin_gradient_invariants]


def _oracle_fwd(q, k, v, scale, causal):
    return oracle.forward_head(q, k, v, scale, causal)


def _oracle_bwd(q, k, v, do, scale, causal):
    return oracle.backward_head(q, k, v, do, scale, causal)


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_pin(pin):
    pin(_oracle_fwd, _oracle_bwd)


# ---------------------------------------------------------------- more pins

def test_rows_sum_to_one():
    rng = np.random.default_rng(1)
    for causal in (False, True):
        q, k, _ = _rand(rng, 40, 8)
        p, _, _ = oracle.row_softmax(oracle.masked_scores(q * 3, k * 3, 0.5, causal))
        assert np.abs(p.sum(1) - 1).max() <= 1e-12
        if causal:
            assert np.all(p[np.triu_indices(40, 1)] == 0.0)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("block", [1, 2, 3, 5, 64])
def test_online_recurrence_equals_full(causal, block):
    """Page "突破单卡显存极限…" §2.1: the blockwise recurrence reproduces the full softmax."""
    rng = np.random.default_rng(2)
    n = 23
    q, k, v = _rand(rng, n, 6)
    block = min(block, n) if block == 64 else block
    o_ref, lse_ref = oracle.forward_head(q * 2, k * 2, v, 0.8, causal)
    o, lse = oracle.online_softmax_forward_head(q * 2, k * 2, v, 0.8, causal, block)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_scalar_brute_force(causal):
    rng = np.random.default_rng(9)
    for n in (1, 2, 5, 8):
        for d in (1, 3, 4):
            q, k, v = _rand(rng, n, d)
            o_ref, lse_ref = oracle.scalar_forward_head(q.tolist(), k.tolist(), v.tolist(), 0.45, causal)
            o, lse = oracle.forward_head(q, k, v, 0.45, causal)
            np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
            np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_row_blocks_equal_unblocked(causal):
    rng = np.random.default_rng(10)
    n = 50
    q, k, v = _rand(rng, n, 4)
    do = rng.standard_normal((n, 4))
    o1, l1 = oracle.forward_head(q, k, v, 0.5, causal)
    o2, l2 = oracle.forward_head(q, k, v, 0.5, causal, row_block=7)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-13)
    g1 = oracle.backward_head(q, k, v, do, 0.5, causal)
    g2 = oracle.backward_head(q, k, v, do, 0.5, causal, row_block=7)
    for a, b in zip(g1, g2):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_row_shares_give_row_gradients_and_the_causal_key_tail(causal):
    """backward_head_rows on a subset of rows: their dQ rows are those of the
    whole head (a row's dQ depends on that row alone), and under the causal
    mask the rows j0 .. N-1 give the complete dK, dV of the keys j0 .. N-1.
    Checked against the whole-head backward, which the autograd and finite
    difference pins above fix; leaving out row j0 must change key j0's
    gradients (so the tail check can fail)."""
    rng = np.random.default_rng(3301)
    n, d = 80, 32
    q, k, v, do = (rng.standard_normal((n, d)) for _ in range(4))
    scale = 1.0 / math.sqrt(d)
    dq, dk, dv = A.backward_head(q, k, v, do, scale, causal)
    rows = np.array([0, 7, 41, 79])
    dq_r, _, _ = A.backward_head_rows(q, k, v, do, scale, causal, rows)
    np.testing.assert_allclose(dq_r, dq[rows], rtol=1e-12, atol=1e-13)
    if not causal:
        return
    j0 = 60
    _, dk_t, dv_t = A.backward_head_rows(q, k, v, do, scale, True, np.arange(j0, n))
    np.testing.assert_allclose(dk_t[j0:], dk[j0:], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dv_t[j0:], dv[j0:], rtol=1e-12, atol=1e-13)
    _, dk_m, dv_m = A.backward_head_rows(q, k, v, do, scale, True, np.arange(j0 + 1, n))
    assert not np.allclose(dk_m[j0], dk[j0], rtol=1e-6, atol=1e-9)
    assert not np.allclose(dv_m[j0], dv[j0], rtol=1e-6, atol=1e-9)


def test_multihead_wrappers_match_heads():
    rng = np.random.default_rng(11)
    q, k, v, do = (rng.standard_normal((2, 3, 10, 4)) for _ in range(4))
    o, lse = oracle.forward(q, k, v, 0.5, True)
    dq, dk, dv = oracle.backward(q, k, v, do, 0.5, True)
    for b in range(2):
        for h in range(3):
            oh, lh = oracle.forward_head(q[b, h], k[b, h], v[b, h], 0.5, True)
            assert np.array_equal(o[b, h], oh) and np.array_equal(lse[b, h], lh)
            gh = oracle.backward_head(q[b, h], k[b, h], v[b, h], do[b, h], 0.5, True)
            assert all(np.array_equal(x[b, h], y) for x, y in zip((dq, dk, dv), gh))


# ---------------------------------------------------------------- planted mistakes

def _mut_bwd(kind):
    def bwd(q, k, v, do, scale, causal):
        s = A.masked_scores(q, k, scale, causal)
        p, _, _ = A.row_softmax(s)
        dv = p.T @ do
        dp = do @ v.T
        dsum = (p * dp).sum(1)
        ds = p * (dp - (0.0 if kind == "no_D" else dsum[:, None]))
        dq = (1.0 if kind == "dq_no_scale" else scale) * (ds @ k)
        dk = scale * ((ds if kind == "dk_transposed" else ds.T) @ q)
        if kind == "dv_transposed":
            dv = p @ do
        if kind == "dq_sign":
            dq = -dq
        return dq, dk, dv
    return bwd


def _mut_fwd(kind):
    def fwd(q, k, v, scale, causal):
        s = float(scale) * (q @ k.T)
        if causal:
            n = q.shape[0]
            j, i = np.meshgrid(np.arange(n), np.arange(n))
            s[(j < i) if kind == "mask_flipped" else (j > i)] = -np.inf
        if kind == "no_scale":
            s = s / float(scale)
        p, m, l = A.row_softmax(s)
        o = p @ v
        lse = m + np.log(l)
        if kind == "lse_log2":
            lse = lse / math.log(2)
        if kind == "lse_max_only":
            lse = m
        return o, lse
    return fwd


@pytest.mark.parametrize("kind", ["mask_flipped", "no_scale", "lse_log2", "lse_max_only"])
def test_planted_forward_mistake_is_caught(kind):
    caught = []
    for pin in PINS:
        try:
            pin(_mut_fwd(kind), _oracle_bwd)
        except (AssertionError, FloatingPointError, ValueError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"planted forward mistake {kind!r} passed every pin"


@pytest.mark.parametrize("kind", ["no_D", "dq_no_scale", "dk_transposed", "dv_transposed", "dq_sign"])
def test_planted_backward_mistake_is_caught(kind):
    caught = []
    for pin in PINS:
        try:
            pin(_oracle_fwd, _mut_bwd(kind))
        except (AssertionError, FloatingPointError, ValueError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"planted backward mistake {kind!r} passed every pin"


# ---------------------------------------------------------------- KV-cache shapes (Nq != Nk)
# Reading (the pages are silent on the mask when Q has fewer rows than K):
# the Nq queries are the last Nq positions of the sequence whose Nk keys are
# cached, so causal query i sees keys j <= i + Nk - Nq.  The pins tie that
# reading to the square case (pinned above) and to closed forms.

def pin_kv_suffix_of_square(fwd):
    """Decoding the last Nq positions gives the last Nq rows of the square causal result."""
    rng = np.random.default_rng(21)
    nk, d = 13, 5
    q, k, v = _rand(rng, nk, d)
    o_full, lse_full = oracle.forward_head(q, k, v, 0.6, True)
    for nq in (1, 2, 5, 13):
        o, lse = fwd(q[nk - nq:], k, v, 0.6, True)
        np.testing.assert_allclose(o, o_full[nk - nq:], rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse, lse_full[nk - nq:], rtol=0, atol=1e-13)


def pin_kv_last_position_sees_all(fwd):
    """A single causal query (the newest position) attends to every cached key."""
    rng = np.random.default_rng(22)
    q, k, v = _rand(rng, 9, 4)
    o_c, lse_c = fwd(q[:1], k, v, 0.9, True)
    o_n, lse_n = fwd(q[:1], k, v, 0.9, False)
    np.testing.assert_allclose(o_c, o_n, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse_c, lse_n, rtol=0, atol=1e-13)


def pin_kv_uniform_prefix_mean(fwd):
    """Q = 0: query i of Nq sees keys 0 .. i + Nk - Nq, so O_i is their V mean and lse_i = ln(count)."""
    rng = np.random.default_rng(23)
    nq, nk, d = 3, 8, 4
    _, k, v = _rand(rng, nk, d)
    q = np.zeros((nq, d))
    o, lse = fwd(q, k, v, 1.3, True)
    cnt = np.arange(nq) + nk - nq + 1
    mean = np.stack([v[:c].mean(0) for c in cnt])
    np.testing.assert_allclose(o, mean, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, np.log(cnt), rtol=0, atol=1e-13)


KV_PINS = [pin_kv_suffix_of_square, pin_kv_last_position_sees_all, pin_kv_uniform_prefix_mean]


@pytest.mark.parametrize("pin", KV_PINS, ids=[p.__name__ for p in KV_PINS])
def test_oracle_kv_pin(pin):
    pin(oracle.forward_head)


@pytest.mark.parametrize("causal", [False, True])
def test_kv_scalar_and_recurrence_agree(causal):
    """Scalar brute force and the blockwise recurrence agree with the vectorised oracle for Nq != Nk."""
    rng = np.random.default_rng(24)
    for nq, nk in ((1, 1), (1, 6), (3, 7), (4, 4), (2, 9)):
        q = rng.standard_normal((nq, 3))
        k = rng.standard_normal((nk, 3))
        v = rng.standard_normal((nk, 2))
        o, lse = oracle.forward_head(q, k, v, 0.7, causal)
        o_s, lse_s = oracle.scalar_forward_head(q.tolist(), k.tolist(), v.tolist(), 0.7, causal)
        np.testing.assert_allclose(o, o_s, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, lse_s, rtol=0, atol=1e-12)
        for block in (1, 2, 5):
            o_b, lse_b = oracle.online_softmax_forward_head(q, k, v, 0.7, causal, block)
            np.testing.assert_allclose(o_b, o, rtol=0, atol=1e-12)
            np.testing.assert_allclose(lse_b, lse, rtol=0, atol=1e-12)


def test_key_split_partials_merge_by_lse():
    """Attention over disjoint key ranges merges exactly: O = sum_s e^(lse_s - lse) O_s,
    lse = ln sum_s e^(lse_s).  This is what makes a split over keys exact."""
    rng = np.random.default_rng(25)
    q = rng.standard_normal((4, 6)) * 2
    k = rng.standard_normal((23, 6)) * 2
    v = rng.standard_normal((23, 5))
    o_ref, lse_ref = oracle.forward_head(q, k, v, 0.5, False)
    parts = [oracle.forward_head(q, k[a:b], v[a:b], 0.5, False) for a, b in ((0, 5), (5, 6), (6, 23))]
    lse = np.logaddexp.reduce(np.stack([p[1] for p in parts]), axis=0)
    o = sum(np.exp(p[1] - lse)[:, None] * p[0] for p in parts)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-13)


def _mut_kv_fwd(kind):
    def fwd(q, k, v, scale, causal):
        s = float(scale) * (q @ k.T)
        nq, nk = q.shape[0], k.shape[0]
        if causal:
            j, i = np.meshgrid(np.arange(nk), np.arange(nq))
            off = {"top_left": 0, "offset_sign": -(nk - nq), "off_by_one": nk - nq - 1}[kind]
            s[j > i + off] = -np.inf
        with np.errstate(invalid="ignore"):
            p, m, l = A.row_softmax(s)
        return p @ v, m + np.log(l)
    return fwd


@pytest.mark.parametrize("kind", ["top_left", "offset_sign", "off_by_one"])
def test_planted_kv_mask_mistake_is_caught(kind):
    caught = []
    for pin in KV_PINS:
        try:
            pin(_mut_kv_fwd(kind))
        except (AssertionError, FloatingPointError, ValueError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"planted KV-cache mask mistake {kind!r} passed every pin"


# ---------------------------------------------------------------- ALiBi (linear position bias)
# Reading (the pages name ALiBi without a formula): a per-head slope m and
# S_ij += -m |pos_i - j| before the softmax, pos_i = i + Nk - Nq the query's
# position.  Pins: closed forms of the geometric weights it gives to equal
# scores, the KV-cache suffix property with the bias, finite differences.

def pin_alibi_causal_geometric(fwd, bwd=None):
    """Q = 0, causal: row i weights key j by r^(i-j), r = e^-m: lse_i = ln((1 - r^(i+1)) / (1 - r))."""
    rng = np.random.default_rng(31)
    n, d, m = 9, 3, 0.37
    _, k, v = _rand(rng, n, d)
    o, lse = fwd(np.zeros((n, d)), k, v, 0.8, True, m)
    r = math.exp(-m)
    for i in range(n):
        w = np.array([r ** (i - j) for j in range(i + 1)])
        np.testing.assert_allclose(o[i], (w[:, None] * v[: i + 1]).sum(0) / w.sum(), rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse[i], math.log((1 - r ** (i + 1)) / (1 - r)), rtol=0, atol=1e-13)


def pin_alibi_noncausal_symmetric(fwd, bwd=None):
    """Q = 0, non-causal: weights r^|i-j| both ways: lse_i = ln(sum_{t<=i} r^t + sum_{1<=t<n-i} r^t)."""
    rng = np.random.default_rng(32)
    n, d, m = 7, 2, 0.9
    _, k, v = _rand(rng, n, d)
    o, lse = fwd(np.zeros((n, d)), k, v, 0.5, False, m)
    r = math.exp(-m)
    for i in range(n):
        w = np.array([r ** abs(i - j) for j in range(n)])
        np.testing.assert_allclose(o[i], (w[:, None] * v).sum(0) / w.sum(), rtol=0, atol=1e-13)
        geo = (1 - r ** (i + 1)) / (1 - r) + r * (1 - r ** (n - 1 - i)) / (1 - r)
        np.testing.assert_allclose(lse[i], math.log(geo), rtol=0, atol=1e-13)


def pin_alibi_kv_suffix(fwd, bwd=None):
    """The bias follows positions: the last Nq rows of the square causal result equal an Nq-query call."""
    rng = np.random.default_rng(33)
    nk, d, m = 11, 4, 0.25
    q, k, v = _rand(rng, nk, d)
    o_full, lse_full = fwd(q, k, v, 0.7, True, m)
    for nq in (1, 4):
        o, lse = fwd(q[nk - nq:], k, v, 0.7, True, m)
        np.testing.assert_allclose(o, o_full[nk - nq:], rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse, lse_full[nk - nq:], rtol=0, atol=1e-13)


def pin_alibi_zero_slope(fwd, bwd=None):
    rng = np.random.default_rng(34)
    q, k, v = _rand(rng, 6, 3)
    for causal in (False, True):
        a, la = fwd(q, k, v, 0.6, causal, 0.0)
        b, lb = oracle.forward_head(q, k, v, 0.6, causal)
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-14)
        np.testing.assert_allclose(la, lb, rtol=0, atol=1e-14)


ALIBI_PINS = [pin_alibi_causal_geometric, pin_alibi_noncausal_symmetric, pin_alibi_kv_suffix, pin_alibi_zero_slope]


def _alibi_fwd(q, k, v, scale, causal, m):
    return oracle.forward_head(q, k, v, scale, causal, alibi_slope=m)


@pytest.mark.parametrize("pin", ALIBI_PINS, ids=[p.__name__ for p in ALIBI_PINS])
def test_oracle_alibi_pin(pin):
    pin(_alibi_fwd)


def test_alibi_finite_differences():
    """The bias is a constant of the inputs: the backward formulas hold unchanged (central differences)."""
    rng = np.random.default_rng(35)
    h = 1e-6
    for causal in (False, True):
        for nq, nk in ((3, 3), (2, 5)):
            if causal and nk < nq:
                continue
            q = rng.standard_normal((nq, 3))
            k = rng.standard_normal((nk, 3))
            v = rng.standard_normal((nk, 2))
            do = rng.standard_normal((nq, 2))
            grads = oracle.backward_head(q, k, v, do, 0.8, causal, alibi_slope=0.45)
            for which, g in enumerate(grads):
                base = [q, k, v]
                fd = np.zeros_like(g)
                for idx in np.ndindex(*g.shape):
                    plus = [x.copy() for x in base]
                    minus = [x.copy() for x in base]
                    plus[which][idx] += h
                    minus[which][idx] -= h
                    lp = float((oracle.forward_head(*plus, 0.8, causal, alibi_slope=0.45)[0] * do).sum())
                    lm = float((oracle.forward_head(*minus, 0.8, causal, alibi_slope=0.45)[0] * do).sum())
                    fd[idx] = (lp - lm) / (2 * h)
                assert np.linalg.norm(fd - g) <= 1e-6 * max(np.linalg.norm(fd), 1e-12), (causal, nq, nk, which)


def _mut_alibi_fwd(kind):
    def fwd(q, k, v, scale, causal, m):
        nq, nk = q.shape[0], k.shape[0]
        s = float(scale) * (q @ k.T)
        j, i = np.meshgrid(np.arange(nk), np.arange(nq))
        pos = i + (0 if kind == "no_shift" else nk - nq)
        dist = {"sign": -np.abs(pos - j), "no_abs": pos - j}.get(kind, np.abs(pos - j))
        s = s - m * dist
        if causal:
            s[j > i + nk - nq] = -np.inf
        p, mx, l = A.row_softmax(s)
        return p @ v, mx + np.log(l)
    return fwd


@pytest.mark.parametrize("kind", ["sign", "no_abs", "no_shift"])
def test_planted_alibi_mistake_is_caught(kind):
    caught = []
    for pin in ALIBI_PINS:
        try:
            pin(_mut_alibi_fwd(kind))
        except (AssertionError, FloatingPointError, ValueError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"planted ALiBi mistake {kind!r} passed every pin"
