"""Pins for the top-K + rest-of-mass form and its divergence, independent of
any implementation.

``impl_c(zb, k) -> TopK`` builds the stored form of float64 rows;
``impl_kl(topk, zq) -> (kl[n], argmax_quant[n], match[n])`` evaluates the
divergence of full quantized rows from it. The expected values come from the
full KL divergence (GSQ-RCO model card, "How it was made" step 5) that the
coarsened one must equal when every token is stored and never exceed
otherwise (a coarsening cannot increase a KL divergence), from the binary KL
closed form at K = 1, from 50-digit decimal arithmetic, and from direct
checks of what "the K most probable tokens" means.
"""
from __future__ import annotations

import math
from decimal import Decimal, localcontext

import numpy as np

import oracle


def _rng(seed):
    return np.random.default_rng(seed)


def _floor(*rows):
    m = max(float(np.abs(r).max()) for r in rows)
    return 64 * np.finfo(np.float64).eps * (1.0 + m)


def _softmax(z):
    e = np.exp(z - z.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def _run(impl_c, impl_kl, zb, zq, k):
    return impl_kl(impl_c(zb, k), zq)


def pin_topk_all_tokens_is_full_kl(impl_c, impl_kl, seed=61):
    """K = V: nothing is coarsened, the rest mass is exactly 0 and the result is
    the full KL of the reference."""
    g = _rng(seed)
    for v in (1, 2, 9, 300):
        zb = g.normal(0, 3.0, (3, v))
        zq = zb + g.normal(0, 0.4, (3, v))
        t = impl_c(zb, v)
        kl, _, _ = impl_kl(t, zq)
        ref = oracle.rows(zb, zq).kl
        if not (np.all(np.asarray(t.rest) == 0.0) and np.all(np.abs(kl - ref) <= 1e-12 * np.abs(ref) + _floor(zb, zq))):
            return False
    return True


def pin_topk_binary_closed_form(impl_c, impl_kl, seed=62):
    """K = 1: the binary KL of the base's top token against the rest,
    p ln(p/q) + (1 - p) ln((1 - p)/(1 - q))."""
    g = _rng(seed)
    zb = g.normal(0, 2.0, (20, 50))
    zq = zb + g.normal(0, 0.7, (20, 50))
    kl, _, _ = _run(impl_c, impl_kl, zb, zq, 1)
    r = np.arange(20)
    i = np.argmax(zb, axis=1)
    p, q = _softmax(zb)[r, i], _softmax(zq)[r, i]
    ref = p * np.log(p / q) + (1 - p) * np.log((1 - p) / (1 - q))
    return bool(np.all(np.abs(kl - ref) <= 1e-10 * np.abs(ref) + _floor(zb, zq)))


def pin_topk_monotone_and_below_full(impl_c, impl_kl, seed=63):
    """Storing one more token refines the partition: KL_K is non-decreasing in K
    and never exceeds the full KL."""
    g = _rng(seed)
    zb = g.normal(0, 2.5, (4, 40))
    zq = zb + g.normal(0, 0.8, (4, 40))
    full = oracle.rows(zb, zq).kl
    prev = np.full(4, -np.inf)
    for k in range(1, 41):
        kl, _, _ = _run(impl_c, impl_kl, zb, zq, k)
        fl = _floor(zb, zq)
        if np.any(kl < prev - fl) or np.any(kl > full + fl):
            return False
        prev = kl
    return True


def _dec_topk_kl(zb, zq, k, digits=50):
    order = sorted(range(len(zb)), key=lambda i: (-float(zb[i]), i))[:k]
    with localcontext() as ctx:
        ctx.prec = digits
        eb = [Decimal(float(x)).exp() for x in zb]
        eq = [Decimal(float(x)).exp() for x in zq]
        sb, sq = sum(eb, Decimal(0)), sum(eq, Decimal(0))
        kl = Decimal(0)
        for i in order:
            p, q = eb[i] / sb, eq[i] / sq
            kl += p * (p.ln() - q.ln())
        others = [i for i in range(len(zb)) if i not in order]
        if others:
            R = sum((eb[i] for i in others), Decimal(0)) / sb
            Q = sum((eq[i] for i in others), Decimal(0)) / sq
            kl += R * (R.ln() - Q.ln())
        return float(kl)


def pin_topk_bruteforce(impl_c, impl_kl, seed=64):
    """50-digit decimal coarsened KL on V <= 8, every K."""
    g = _rng(seed)
    for c in range(16):
        v = int(g.integers(1, 9))
        zb = g.normal(0, [0.5, 2.0, 6.0, 20.0][c % 4], v)
        zq = zb + g.normal(0, [0.05, 0.5, 2.0][c % 3], v)
        if c % 5 == 0 and v > 2:
            zb[1] = zb[0]                     # a tie inside or at the edge of the stored set
        for k in range(1, v + 1):
            kl, _, _ = _run(impl_c, impl_kl, zb[None], zq[None], k)
            ref = _dec_topk_kl(zb, zq, k)
            if abs(kl[0] - ref) > 1e-12 * abs(ref) + _floor(zb, zq):
                return False
    return True


def pin_compress_selects_most_probable(impl_c, impl_kl, seed=65):
    """Every stored token outranks every other one, ranking by value then lowest
    index; the stored list is in rank order; +0 and -0 are equal."""
    g = _rng(seed)
    v, k = 200, 17
    zb = np.round(g.normal(0, 2.0, (6, v)), 1)          # many exact ties
    zb[0, :] = 0.0
    zb[0, 3::7] = -0.0                                   # signed zeros only
    zb[1, 150:] = 9.0                                    # a run of equal maxima at the end
    t = impl_c(zb, k)
    for r in range(6):
        sel = [int(i) for i in t.idx[r]]
        key = lambda i: (-float(zb[r, i]) + 0.0, i)  # noqa: E731
        if sel != sorted(sel, key=key):
            return False
        worst_in = max(key(i) for i in sel)
        others = set(range(v)) - set(sel)
        if len(set(sel)) != k or any(key(i) < worst_in for i in others):
            return False
    return True


def pin_compress_mass_sums_to_one(impl_c, impl_kl, seed=66):
    """Stored probabilities plus the rest mass sum to one; the rest is positive
    whenever some token is left out."""
    g = _rng(seed)
    zb = g.normal(0, 4.0, (5, 1000))
    t = impl_c(zb, 128)
    tot = [math.fsum(np.exp(np.asarray(t.logp[r], np.float64)).tolist()) + float(t.rest[r]) for r in range(5)]
    return bool(np.all(np.abs(np.array(tot) - 1.0) <= 1e-13)) and bool(np.all(np.asarray(t.rest) > 0))


def pin_topk_identical_rows_and_match(impl_c, impl_kl, seed=67):
    """A quantized row equal to the base row diverges by 0; the top-1 match
    compares the quantized argmax (lowest index) with the first stored token."""
    g = _rng(seed)
    zb = g.normal(0, 3.0, (6, 500))
    zq = zb.copy()
    zq[3] = zq[3] + g.normal(0, 3.0, 500)
    zq[4, :] = zq[4].max() + 1.0                          # constant row: argmax 0
    kl, am, match = _run(impl_c, impl_kl, zb, zq, 64)
    ok = bool(np.all(np.abs(kl[[0, 1, 2, 5]]) <= _floor(zb, zq)))
    return ok and np.array_equal(am, np.argmax(zq, axis=1)) and np.array_equal(
        match, (np.argmax(zq, axis=1) == np.argmax(zb, axis=1)).astype(np.uint8))


ALL_PINS = [pin_topk_all_tokens_is_full_kl, pin_topk_binary_closed_form, pin_topk_monotone_and_below_full,
            pin_topk_bruteforce, pin_compress_selects_most_probable, pin_compress_mass_sums_to_one,
            pin_topk_identical_rows_and_match]


# ---- gradient of KL_K with respect to the quantized logits ----
# impl_g(topk, zq, scale) -> g [n, V]

def pin_topk_grad_all_tokens_is_q_minus_p(impl_c, impl_g, seed=71):
    """K = V: the gradient of the full KL, q - p (softmax closed form)."""
    g = _rng(seed)
    zb = g.normal(0, 2.0, (3, 60))
    zq = zb + g.normal(0, 0.5, (3, 60))
    gr = impl_g(impl_c(zb, 60), zq, 1.0)
    return bool(np.all(np.abs(gr - (_softmax(zq) - _softmax(zb))) <= 1e-14))


def pin_topk_grad_central_difference(impl_c, impl_g, seed=72):
    """Central differences of the 50-digit coarsened KL (stored form fixed) in
    each quant logit, V <= 7, every K."""
    g = _rng(seed)
    for c in range(6):
        v = int(g.integers(2, 8))
        zb = g.normal(0, [1.0, 3.0][c % 2], v)
        zq = zb + g.normal(0, 0.6, v)
        for k in range(1, v + 1):
            gr = impl_g(impl_c(zb[None], k), zq[None], 1.0)[0]
            for j in range(v):
                up, dn = zq.copy(), zq.copy()
                up[j] += 1e-6
                dn[j] -= 1e-6
                fd = (_dec_topk_kl(zb, up, k) - _dec_topk_kl(zb, dn, k)) / (up[j] - dn[j])
                if abs(gr[j] - fd) > 1e-8:
                    return False
    return True


def pin_topk_grad_directional_derivative(impl_c, impl_g, seed=73):
    """Directional derivatives of KL_K on V = 2000, K = 64, with the stored form
    held fixed: (KL_K(zq + h u) - KL_K(zq - h u)) / 2h = g . u."""
    g = _rng(seed)
    zb = g.normal(0, 3.0, (3, 2000))
    zq = zb + g.normal(0, 0.4, (3, 2000))
    t = impl_c(zb, 64)
    gr = impl_g(t, zq, 1.0)
    from oracle import topk as otk
    h = 1e-4
    for r in range(3):
        u = g.normal(0, 1.0, 2000)
        tr = otk.TopK(t.idx[r:r + 1], t.logp[r:r + 1], np.asarray(t.rest)[r:r + 1])
        kp = otk.kl_topk(tr, (zq[r] + h * u)[None], oracle.rows(zq[r:r + 1] + h * u, zq[r:r + 1] + h * u).lse_base).kl[0]
        km = otk.kl_topk(tr, (zq[r] - h * u)[None], oracle.rows(zq[r:r + 1] - h * u, zq[r:r + 1] - h * u).lse_base).kl[0]
        fd = (kp - km) / (2 * h)
        if abs(fd - float(gr[r] @ u)) > 1e-7 * (1 + abs(fd)):
            return False
    return True


def pin_topk_grad_sums_to_zero_and_scales(impl_c, impl_g, seed=74):
    """With stored mass P + R = 1 the gradient rows sum to zero; it is linear
    in the row weight."""
    g = _rng(seed)
    zb = g.normal(0, 3.0, (4, 800))
    zq = zb + g.normal(0, 1.0, (4, 800))
    t = impl_c(zb, 32)
    a = impl_g(t, zq, 1.0)
    b = impl_g(t, zq, -2.5)
    return (bool(np.all(np.abs([math.fsum(x.tolist()) for x in a]) <= 1e-13))
            and bool(np.all(np.abs(b + 2.5 * a) <= 1e-15 + 1e-14 * np.abs(a))))


GRAD_PINS = [pin_topk_grad_all_tokens_is_q_minus_p, pin_topk_grad_central_difference,
             pin_topk_grad_directional_derivative, pin_topk_grad_sums_to_zero_and_scales]
