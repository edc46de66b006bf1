"""Pins for the token-conditioned metrics, independent of any implementation.

Row pins take ``impl(zb, zq, tokens) -> (logp_base[n], logp_quant[n], dp[n],
state[n])`` on float64 [n, V] rows; summary pins take ``impl_sum(logp_base,
logp_quant, dp, state) -> object`` with the fields of a token summary. The
expected values come from the definition of a softmax probability
(p_t = e^{z_t} / sum_j e^{z_j}), from closed forms derived from it, from
50-digit decimal arithmetic, and from identities that tie the token metrics to
the KL divergence: averaging log p_base(t) - log p_quant(t) over t drawn from
the base distribution gives KL(P_base || Q_quant) (GSQ-RCO model card, "How it
was made" step 5), and the probabilities of all tokens sum to one.
"""
from __future__ import annotations

import math
from decimal import Decimal, localcontext

import numpy as np

from oracle.bruteforce import bruteforce


def _rng(seed):
    return np.random.default_rng(seed)


def _close(a, b, rel, abs_=0.0):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return bool(np.all(np.abs(a - b) <= np.maximum(rel * np.abs(b), abs_)))


def _floor(*rows):
    """Absolute rounding floor of a float64 log-probability: z_t - lse with
    lse ~ max|z| carries ~eps64 * max|z| of rounding."""
    m = max(float(np.abs(r).max()) for r in rows)
    return 16 * np.finfo(np.float64).eps * (1.0 + m)


def _dec_logp(z, t, digits=50):
    """ln(e^{z_t} / sum_j e^{z_j}) in 50-digit decimal arithmetic, no shift."""
    with localcontext() as ctx:
        ctx.prec = digits
        e = [Decimal(float(v)).exp() for v in z]
        return float((e[t] / sum(e, Decimal(0))).ln())


def pin_tok_uniform_rows(impl, seed=21):
    """Constant rows: every token has p = 1/V, so log p = -ln V and dp = 0."""
    ok = True
    for v in (1, 2, 7, 1000):
        zb = np.full((3, v), 2.5)
        zq = np.full((3, v), -11.0)
        t = np.array([0, v - 1, v // 2])
        lpb, lpq, dp, st = impl(zb, zq, t)
        ok &= _close(lpb, -math.log(v), 0, 1e-13) and _close(lpq, -math.log(v), 0, 1e-13)
        ok &= _close(dp, 0.0, 0, 1e-15) and bool(np.all(st == 1))
    return ok


def pin_tok_two_token_closed_form(impl, seed=22):
    """V = 2: log p_0 = -ln(1 + e^{z_1 - z_0}), log p_1 = -ln(1 + e^{z_0 - z_1})."""
    g = _rng(seed)
    zb = g.normal(0, 3.0, (40, 2))
    zq = g.normal(0, 3.0, (40, 2))
    t = g.integers(0, 2, 40)
    lpb, lpq, dp, _ = impl(zb, zq, t)
    o = 1 - t
    r = np.arange(40)
    eb = -np.log1p(np.exp(zb[r, o] - zb[r, t]))
    eq = -np.log1p(np.exp(zq[r, o] - zq[r, t]))
    return (_close(lpb, eb, 1e-12, _floor(zb)) and _close(lpq, eq, 1e-12, _floor(zq))
            and _close(dp, np.exp(eq) - np.exp(eb), 1e-10, 1e-15))


def pin_tok_bruteforce(impl, seed=23):
    """Agreement with 50-digit decimal log-probabilities on V <= 8."""
    g = _rng(seed)
    for c in range(30):
        v = int(g.integers(1, 9))
        s = [0.5, 2.0, 8.0, 30.0][c % 4]
        zb = g.normal(0, s, v)
        zq = zb + g.normal(0, [0.01, 0.3, 2.0][c % 3], v)
        t = int(g.integers(0, v))
        lpb, lpq, dp, st = impl(zb[None], zq[None], np.array([t]))
        eb, eq = _dec_logp(zb, t), _dec_logp(zq, t)
        if not (_close(lpb[0], eb, 1e-12, _floor(zb)) and _close(lpq[0], eq, 1e-12, _floor(zq))):
            return False
        if not _close(dp[0], math.exp(eq) - math.exp(eb), 1e-9, 1e-14) or st[0] != 1:
            return False
    return True


def pin_tok_enumeration(impl, seed=24):
    """One row scored at every token: the probabilities sum to one, the dp sum
    to zero, and sum_t p_base(t) (log p_base(t) - log p_quant(t)) is the KL
    divergence, checked against the 50-digit brute force."""
    g = _rng(seed)
    ok = True
    for v, s in ((5, 1.0), (8, 6.0), (300, 3.0)):
        zb = g.normal(0, s, v)
        zq = zb + g.normal(0, 0.4, v)
        t = np.arange(v)
        lpb, lpq, dp, _ = impl(np.tile(zb, (v, 1)), np.tile(zq, (v, 1)), t)
        p = np.exp(lpb)
        ok &= abs(math.fsum(p.tolist()) - 1.0) <= 1e-12
        ok &= abs(math.fsum(np.exp(lpq).tolist()) - 1.0) <= 1e-12
        ok &= abs(math.fsum(dp.tolist())) <= 1e-12
        if v <= 8:
            ref = float(bruteforce(zb, zq)[0])
            ok &= abs(math.fsum((p * (lpb - lpq)).tolist()) - ref) <= 1e-12 + _floor(zb, zq)
    return bool(ok)


def pin_tok_bump_closed_form(impl, seed=25):
    """zq = zb + delta at the scored token t only: log q_t - log p_t =
    delta - ln(1 + p_t (e^delta - 1)), and dp has the sign of delta."""
    g = _rng(seed)
    n, v = 10, 3000
    zb = g.normal(0, 3.0, (n, v))
    t = g.integers(0, v, n)
    delta = g.normal(0, 2.0, n)
    zq = zb.copy()
    r = np.arange(n)
    zq[r, t] += delta
    lpb, lpq, dp, _ = impl(zb, zq, t)
    pt = np.exp(zb[r, t] - zb.max(axis=1)) / np.exp(zb - zb.max(axis=1, keepdims=True)).sum(axis=1)
    ref = delta - np.log1p(pt * np.expm1(delta))
    return _close(lpq - lpb, ref, 1e-9, _floor(zb, zq)) and bool(np.all(np.sign(dp) == np.sign(delta)))


def pin_tok_shift_invariance(impl, seed=26):
    """Adding a constant to a whole row changes no probability."""
    g = _rng(seed)
    zb = g.normal(0, 3.0, (6, 800))
    zq = zb + g.normal(0, 0.3, (6, 800))
    t = g.integers(0, 800, 6)
    a = impl(zb, zq, t)
    b = impl(zb - 40.5, zq + 17.25, t)
    fl = _floor(zb, zq) * 8
    return all(_close(x, y, 1e-10, fl) for x, y in zip(a[:3], b[:3]))


def pin_tok_states(impl, seed=27):
    """Negative ids are not scored (state 0), ids >= V are invalid (state 2),
    every other id is scored (state 1); unscored rows carry NaN."""
    g = _rng(seed)
    v = 50
    t = np.array([-7, -1, 0, v - 1, v, v + 1000, 25])
    zb = g.normal(0, 2.0, (7, v))
    zq = zb + 0.1
    lpb, lpq, dp, st = impl(zb, zq, t)
    want = np.array([0, 0, 1, 1, 2, 2, 1])
    sc = want == 1
    return (np.array_equal(st, want) and bool(np.all(np.isnan(lpb[~sc]))) and bool(np.all(np.isnan(dp[~sc])))
            and bool(np.all(np.isfinite(lpb[sc]))) and bool(np.all(np.isfinite(lpq[sc]))))


ROW_PINS = [pin_tok_uniform_rows, pin_tok_two_token_closed_form, pin_tok_bruteforce, pin_tok_enumeration,
            pin_tok_bump_closed_form, pin_tok_shift_invariance, pin_tok_states]


def pin_sum_geometric_mean(impl_sum):
    """Probabilities 1/2 and 1/8: perplexity = 1 / geometric mean = 4; with the
    quantized model at 1/4 and 1/4 it is 4 too, so the ratio is 1."""
    lpb = np.log([0.5, 0.125])
    lpq = np.log([0.25, 0.25])
    dp = np.array([0.25 - 0.5, 0.25 - 0.125])
    s = impl_sum(lpb, lpq, dp, np.array([1, 1], np.uint8))
    return (s.n_scored == 2 and abs(s.ppl_base - 4.0) <= 1e-14 and abs(s.ppl_quant - 4.0) <= 1e-14
            and abs(s.ppl_ratio - 1.0) <= 1e-14 and abs(s.dp_mean - (-0.125 / 2)) <= 1e-16
            and abs(s.dp_rms - math.sqrt((0.0625 + 0.015625) / 2)) <= 1e-16)


def pin_sum_excludes_unscored(impl_sum, seed=28):
    """Rows that are not scored or invalid change nothing but the counts."""
    g = _rng(seed)
    lpb = -g.exponential(2.0, 50)
    lpq = lpb + g.normal(0, 0.1, 50)
    dp = np.exp(lpq) - np.exp(lpb)
    st = np.ones(50, np.uint8)
    a = impl_sum(lpb, lpq, dp, st)
    lpb2 = np.concatenate([lpb, [np.nan, np.nan, 5.0]])
    lpq2 = np.concatenate([lpq, [np.nan, np.nan, -9.0]])
    dp2 = np.concatenate([dp, [np.nan, np.nan, 0.7]])
    st2 = np.concatenate([st, np.array([0, 2, 0], np.uint8)])
    b = impl_sum(lpb2, lpq2, dp2, st2)
    same = all(getattr(a, f) == getattr(b, f) for f in ("ppl_base", "ppl_quant", "ppl_ratio", "dp_mean", "dp_rms"))
    return same and a.n_scored == 50 and b.n_scored == 50 and b.n_invalid == 1 and a.n_invalid == 0


def pin_sum_ratio_is_exp_of_mean_gap(impl_sum, seed=29):
    """ppl_quant / ppl_base = exp(mean(log p_base - log p_quant))."""
    g = _rng(seed)
    lpb = -g.exponential(3.0, 200)
    lpq = lpb + g.normal(0, 0.5, 200)
    s = impl_sum(lpb, lpq, np.exp(lpq) - np.exp(lpb), np.ones(200, np.uint8))
    ref = math.exp(math.fsum((lpb - lpq).tolist()) / 200)
    return abs(s.ppl_ratio - ref) <= 1e-12 * ref and abs(s.ppl_quant - math.exp(-math.fsum(lpq.tolist()) / 200)) <= 1e-12 * s.ppl_quant


def pin_sum_overflowing_perplexities(impl_sum):
    """Mean negative log-likelihoods of 800 and 801 nats: both perplexities lie
    past the largest double (709.78 nats), +inf in float64, while their ratio
    is exp(-1) exactly as the definition gives it (a ratio of the two
    exponentials, e^801 / e^800 inverted)."""
    lpb = np.array([-801.0, -801.0])
    lpq = np.array([-800.0, -800.0])
    s = impl_sum(lpb, lpq, np.zeros(2), np.ones(2, np.uint8))
    return s.ppl_base == math.inf and s.ppl_quant == math.inf and abs(s.ppl_ratio - math.exp(-1.0)) <= 1e-15


def pin_sum_no_scored_rows(impl_sum):
    """No scored row: counts are zero and every mean is NaN."""
    s = impl_sum(np.array([np.nan]), np.array([np.nan]), np.array([np.nan]), np.array([0], np.uint8))
    return s.n_scored == 0 and all(math.isnan(getattr(s, f)) for f in ("ppl_base", "ppl_quant", "dp_mean", "dp_rms"))


SUM_PINS = [pin_sum_geometric_mean, pin_sum_excludes_unscored, pin_sum_ratio_is_exp_of_mean_gap,
            pin_sum_overflowing_perplexities, pin_sum_no_scored_rows]
