"""Pins for a KL/top-1 implementation, independent of any implementation.

Each pin takes ``impl(zb, zq) -> (kl[n], argmax_base[n], argmax_quant[n])`` on
float64 [n, V] arrays and returns True when the implementation satisfies what
the definition fixes. The expected values come from closed forms derived here
from KL(P || Q) = sum_i p_i log(p_i / q_i) with P the base softmax and Q the
quantized one (GSQ-RCO model card, "How it was made" step 5), from invariants
of that definition, from a 50-digit brute force, and from NumPy's documented
first-occurrence argmax. The test suite runs every pin against the oracles and
also against deliberately broken implementations, to show the pins bite.
"""
from __future__ import annotations

import math

import numpy as np

from oracle.bruteforce import bruteforce


def _rng(seed):
    return np.random.default_rng(seed)


def _close(a, b, rel, abs_=0.0):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return bool(np.all(np.abs(a - b) <= np.maximum(rel * np.abs(b), abs_)))


def _f64_floor(zb, zq):
    """Absolute rounding floor of a float64 evaluation: the textbook formula
    subtracts two log-normalisers of size ~max|z|, so its error is a small
    multiple of eps64 * max|z| per row, far below any float32 tolerance."""
    m = np.maximum(np.abs(zb).max(axis=-1), np.abs(zq).max(axis=-1))
    return 16 * np.finfo(np.float64).eps * (1.0 + m)


def _softmax_rows(z):
    z = z - z.max(axis=1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=1, keepdims=True)


def pin_bruteforce(impl, n_cases=40, seed=1):
    """Agreement with 50-digit decimal arithmetic on V <= 8 (random + adversarial)."""
    g = _rng(seed)
    cases = []
    for c in range(n_cases):
        v = int(g.integers(1, 9))
        scale = [0.3, 1.0, 3.0, 10.0, 40.0][c % 5]
        zb = g.normal(0, scale, v)
        zq = zb + g.normal(0, [1e-3, 0.05, 0.5, 2.0][c % 4], v)
        cases.append((zb, zq))
    # adversarial: ties, large offsets, one dominant token, reversed order
    cases.append((np.array([5.0, 5.0, 1.0]), np.array([1.0, 5.0, 5.0])))
    cases.append((np.array([80.0, 79.0, -30.0, 0.0]), np.array([-40.0, 79.5, 81.0, 0.0])))
    cases.append((np.array([0.0, 0.0, 0.0, 0.0]), np.array([3.0, 0.0, 0.0, -3.0])))
    cases.append((np.array([12.0, 0.1, -0.1]), np.array([12.0, 0.1, -0.1]) + np.array([0.0, 1e-6, -1e-6])))
    for zb, zq in cases:
        kl, ib, iq = impl(zb[None], zq[None])
        ref, rb, rq = bruteforce(zb, zq)
        ref = float(ref)
        # float64 evaluation of the textbook formula subtracts two log-normalisers of
        # size ~max|z|; its rounding is then ~eps64 * max|z| in absolute terms
        if not _close(kl[0], ref, 1e-12, _f64_floor(zb, zq)):
            return False
        if int(ib[0]) != rb or int(iq[0]) != rq:
            return False
    return True


def pin_identical_rows_zero(impl, seed=2):
    """KL(p || p) = 0: identical rows give exactly zero."""
    g = _rng(seed)
    z = g.normal(0, 4.0, (6, 1000))
    kl, ib, iq = impl(z, z.copy())
    return bool(np.all(kl == 0.0)) and bool(np.all(ib == iq))


def pin_nonnegative(impl, seed=3):
    """Gibbs' inequality: KL >= 0 (up to float64 rounding)."""
    g = _rng(seed)
    zb = g.normal(0, 3.0, (20, 500))
    zq = zb + g.normal(0, 0.3, (20, 500))
    kl, _, _ = impl(zb, zq)
    return bool(np.all(kl >= -1e-12)) and bool(np.all(kl > 0))


def pin_shift_invariance(impl, seed=4):
    """Adding a constant to every logit of either row leaves KL and argmax unchanged."""
    g = _rng(seed)
    zb = g.normal(0, 3.0, (8, 700))
    zq = zb + g.normal(0, 0.2, (8, 700))
    kl0, ib0, iq0 = impl(zb, zq)
    kl1, ib1, iq1 = impl(zb + 7.25, zq - 13.5)
    return _close(kl1, kl0, 1e-9, _f64_floor(zb, zq) + 1e-13) and np.array_equal(ib0, ib1) and np.array_equal(iq0, iq1)


def pin_permutation_invariance(impl, seed=5):
    """A joint permutation of the vocabulary permutes the argmaxes and keeps KL."""
    g = _rng(seed)
    zb = g.normal(0, 3.0, (5, 300))
    zq = zb + g.normal(0, 0.5, (5, 300))
    perm = g.permutation(300)
    kl0, ib0, iq0 = impl(zb, zq)
    kl1, ib1, iq1 = impl(zb[:, perm], zq[:, perm])
    inv = np.argsort(perm)
    return _close(kl1, kl0, 1e-10, _f64_floor(zb, zq)) and np.array_equal(inv[ib0], ib1) and np.array_equal(inv[iq0], iq1)


def pin_two_token_closed_form(impl, seed=6):
    """V = 2: KL = p ln(p/q) + (1-p) ln((1-p)/(1-q)), p = sigmoid(zb0 - zb1)."""
    g = _rng(seed)
    zb = g.normal(0, 2.0, (30, 2))
    zq = g.normal(0, 2.0, (30, 2))
    kl, _, _ = impl(zb, zq)
    p = 1.0 / (1.0 + np.exp(-(zb[:, 0] - zb[:, 1])))
    q = 1.0 / (1.0 + np.exp(-(zq[:, 0] - zq[:, 1])))
    ref = p * np.log(p / q) + (1 - p) * np.log((1 - p) / (1 - q))
    return _close(kl, ref, 1e-11, _f64_floor(zb, zq))


def pin_bump_closed_form(impl, seed=7):
    """zq = zb + delta * e_k: KL = -delta p_k + ln(1 - p_k + p_k e^delta)."""
    g = _rng(seed)
    n, v = 12, 5000
    zb = g.normal(0, 3.0, (n, v))
    k = g.integers(0, v, n)
    delta = g.normal(0, 2.0, n)
    zq = zb.copy()
    zq[np.arange(n), k] += delta
    kl, _, _ = impl(zb, zq)
    pk = _softmax_rows(zb)[np.arange(n), k]
    ref = -delta * pk + np.log1p(pk * np.expm1(delta))
    return _close(kl, ref, 1e-9, _f64_floor(zb, zq))


def pin_swap_closed_form(impl, seed=8):
    """zq = zb with entries j, k swapped: KL = (p_j - p_k)(zb_j - zb_k)."""
    g = _rng(seed)
    n, v = 12, 4000
    zb = g.normal(0, 4.0, (n, v))
    j = g.integers(0, v, n)
    k = (j + g.integers(1, v, n)) % v
    zq = zb.copy()
    r = np.arange(n)
    zq[r, j], zq[r, k] = zb[r, k], zb[r, j]
    kl, _, _ = impl(zb, zq)
    p = _softmax_rows(zb)
    ref = (p[r, j] - p[r, k]) * (zb[r, j] - zb[r, k])
    return _close(kl, ref, 1e-9, _f64_floor(zb, zq))


def pin_uniform_quant(impl, seed=9):
    """Constant quant row: KL = ln V - H(p)."""
    g = _rng(seed)
    zb = g.normal(0, 2.0, (6, 900))
    zq = np.full_like(zb, 0.5)
    kl, _, iq = impl(zb, zq)
    p = _softmax_rows(zb)
    ref = math.log(900) + np.sum(p * np.log(p), axis=1)
    return _close(kl, ref, 1e-10, _f64_floor(zb, zq)) and bool(np.all(iq == 0))


def pin_uniform_base(impl, seed=10):
    """Constant base row: KL = -ln V - (1/V) sum_i ln q_i."""
    g = _rng(seed)
    zq = g.normal(0, 2.0, (6, 900))
    zb = np.full_like(zq, -1.0)
    kl, ib, _ = impl(zb, zq)
    q = _softmax_rows(zq)
    ref = -math.log(900) - np.mean(np.log(q), axis=1)
    return _close(kl, ref, 1e-10, _f64_floor(zb, zq)) and bool(np.all(ib == 0))


def pin_argmax_lowest_index(impl, seed=11):
    """Planted exact ties: the argmax is the lowest tied index (NumPy's rule)."""
    g = _rng(seed)
    n, v = 16, 257
    zb = g.normal(0, 1.0, (n, v))
    zq = zb + g.normal(0, 0.1, (n, v))
    for r in range(n):
        idx = np.sort(g.choice(v, size=2 + r % 3, replace=False))
        zb[r, idx] = 9.0
        zq[r, idx[1:]] = 9.5   # quant ties exclude the base's first index
    zb[0, 0] = zb[0, -1] = 20.0   # ties at the row's two ends
    _, ib, iq = impl(zb, zq)
    return np.array_equal(ib, np.argmax(zb, axis=1)) and np.array_equal(iq, np.argmax(zq, axis=1))


def flat_rows_closed_form(vocab, raised_b, raised_q):
    """KL, lse_base and lse_quant of two rows of `vocab` logits that are 0 but
    at a few tokens ({index: logit}). Z = (V - m) + sum of e^z over the m
    raised tokens; the flat tokens have zb_i = zq_i = 0, so only the raised
    tokens of either row enter sum_i p_i (zb_i - zq_i), and
    KL = that sum + log(Zq / Zb), with p_i = e^{zb_i} / Zb."""
    zb = (vocab - len(raised_b)) + sum(math.exp(v) for v in raised_b.values())
    zq = (vocab - len(raised_q)) + sum(math.exp(v) for v in raised_q.values())
    dz = (len(raised_b) - len(raised_q)) + sum(math.exp(v) for v in raised_q.values()) \
        - sum(math.exp(v) for v in raised_b.values())  # Zq - Zb, formed without V
    kl = math.log1p(dz / zb)
    for i in set(raised_b) | set(raised_q):
        xb, xq = raised_b.get(i, 0.0), raised_q.get(i, 0.0)
        kl += math.exp(xb) / zb * (xb - xq)
    return kl, math.log(zb), math.log(zq)


def pin_flat_rows_closed_form(impl):
    """Rows flat (0) but for a few raised tokens: KL against the closed form;
    argmaxes at the largest logit, the lowest index among equal ones (a row
    whose raised tokens lie below 0 has its maximum 0 at the first flat one)."""
    def top(raised, v):
        m = max(0.0, max(raised.values()))
        return min(i for i in range(v) if raised.get(i, 0.0) == m)
    for v in (1001, 50000):
        for rb, rq in (({0: 3.0, v - 2: 20.0}, {0: 2.5, v - 2: 18.0}),
                       ({0: 3.0, v - 2: 20.0}, {0: 2.5, v - 3: 18.0}),
                       ({0: -4.0, 5: -1.0}, {1: 7.0, 2: 7.0})):
            zb = np.zeros((1, v))
            zq = np.zeros((1, v))
            for i, x in rb.items():
                zb[0, i] = x
            for i, x in rq.items():
                zq[0, i] = x
            kl, ib, iq = impl(zb, zq)
            ref = flat_rows_closed_form(v, rb, rq)[0]
            if not (_close(kl, [ref], 1e-9, _f64_floor(zb, zq)) and ib[0] == top(rb, v) and iq[0] == top(rq, v)):
                return False
    return True


ALL_PINS = [
    pin_bruteforce, pin_identical_rows_zero, pin_nonnegative, pin_shift_invariance,
    pin_permutation_invariance, pin_two_token_closed_form, pin_bump_closed_form,
    pin_swap_closed_form, pin_uniform_quant, pin_uniform_base, pin_argmax_lowest_index,
    pin_flat_rows_closed_form,
]
