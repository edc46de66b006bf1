"""Pins for the gradient of KL(P_base || Q_quant) with respect to the quantized
logits, independent of any implementation.

Each pin takes ``impl(zb, zq, scale) -> g`` on float64 [n, V] rows and returns
True when the implementation satisfies what the derivative of the KL
divergence (GSQ-RCO model card, "How it was made" steps 5 and 7) fixes. The
strongest pins differentiate the divergence itself numerically: a central
difference of the 50-digit decimal brute force, and directional derivatives of
the float64 KL reference, so a wrong formula for the gradient cannot agree
with them.
"""
from __future__ import annotations

import math

import numpy as np

import oracle
from oracle.bruteforce import bruteforce


def _rng(seed):
    return np.random.default_rng(seed)


def _close(a, b, rel, abs_=0.0):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return bool(np.all(np.abs(a - b) <= np.maximum(rel * np.abs(b), abs_)))


def pin_grad_finite_difference_bruteforce(impl, seed=41):
    """Central differences of the 50-digit KL in each quant logit, V <= 6."""
    g = _rng(seed)
    for c in range(12):
        v = int(g.integers(1, 7))
        zb = g.normal(0, [0.5, 2.0, 6.0][c % 3], v)
        zq = zb + g.normal(0, [0.05, 0.5, 2.0][c % 3], v)
        gr = impl(zb[None], zq[None], 1.0)[0]
        for i in range(v):
            up, dn = zq.copy(), zq.copy()
            up[i] += 1e-6
            dn[i] -= 1e-6
            h2 = up[i] - dn[i]                     # the step actually taken
            fd = float(bruteforce(zb, up)[0] - bruteforce(zb, dn)[0]) / h2
            if abs(gr[i] - fd) > 1e-9:
                return False
    return True


def pin_grad_directional_derivative(impl, seed=42):
    """(KL(zq + h u) - KL(zq - h u)) / 2h = g . u for random directions u,
    with the float64 KL reference; V in the thousands."""
    g = _rng(seed)
    n, v = 6, 3000
    zb = g.normal(0, 3.0, (n, v))
    zq = zb + g.normal(0, 0.3, (n, v))
    gr = impl(zb, zq, 1.0)
    h = 1e-4
    for r in range(n):
        u = g.normal(0, 1.0, v)
        kp = oracle.rows(zb[r:r + 1], (zq[r] + h * u)[None]).kl[0]
        km = oracle.rows(zb[r:r + 1], (zq[r] - h * u)[None]).kl[0]
        fd = (kp - km) / (2 * h)
        if abs(fd - float(gr[r] @ u)) > 1e-7 * (1 + abs(fd)):
            return False
    return True


def pin_grad_sums_to_zero(impl, seed=43):
    """Both distributions sum to one, so every row of the gradient sums to zero."""
    g = _rng(seed)
    zb = g.normal(0, 4.0, (5, 2000))
    zq = zb + g.normal(0, 1.0, (5, 2000))
    gr = impl(zb, zq, 1.0)
    return bool(np.all(np.abs([math.fsum(row.tolist()) for row in gr]) <= 1e-13))


def pin_grad_identical_rows_zero(impl, seed=44):
    g = _rng(seed)
    z = g.normal(0, 4.0, (4, 700))
    return bool(np.all(impl(z, z.copy(), 1.0) == 0.0))


def pin_grad_two_token_closed_form(impl, seed=45):
    """V = 2: g_0 = sigmoid(zq_0 - zq_1) - sigmoid(zb_0 - zb_1) = -g_1."""
    g = _rng(seed)
    zb = g.normal(0, 2.0, (30, 2))
    zq = g.normal(0, 2.0, (30, 2))
    gr = impl(zb, zq, 1.0)
    sig = lambda x: 1.0 / (1.0 + np.exp(-x))  # noqa: E731
    ref = sig(zq[:, 0] - zq[:, 1]) - sig(zb[:, 0] - zb[:, 1])
    return _close(gr[:, 0], ref, 1e-12, 1e-15) and _close(gr[:, 1], -ref, 1e-12, 1e-15)


def pin_grad_uniform_quant(impl, seed=46):
    """Constant quant row: g_i = 1/V - p_i."""
    g = _rng(seed)
    v = 500
    zb = g.normal(0, 2.0, (3, v))
    zq = np.full_like(zb, 7.0)
    gr = impl(zb, zq, 1.0)
    p = np.exp(zb - zb.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    return _close(gr, 1.0 / v - p, 1e-12, 1e-16)


def pin_grad_scale_and_shift(impl, seed=47):
    """The gradient is linear in the row weight and unchanged by adding a
    constant to either row."""
    g = _rng(seed)
    zb = g.normal(0, 3.0, (4, 900))
    zq = zb + g.normal(0, 0.5, (4, 900))
    a = impl(zb, zq, 1.0)
    b = impl(zb, zq, -0.375)
    c = impl(zb + 11.5, zq - 30.25, 1.0)
    return _close(b, -0.375 * a, 1e-15, 1e-300) and _close(c, a, 1e-9, 1e-14)


ALL_PINS = [pin_grad_finite_difference_bruteforce, pin_grad_directional_derivative, pin_grad_sums_to_zero,
            pin_grad_identical_rows_zero, pin_grad_two_token_closed_form, pin_grad_uniform_quant,
            pin_grad_scale_and_shift]
