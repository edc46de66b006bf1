"""The token-metric oracle against its pins, and mutants that the pins reject."""
from __future__ import annotations

import math
import sys

import numpy as np
import pytest

import oracle
from oracle import tokens as otok

from tests import pins_tokens as pt


def oracle_tok(zb, zq, t):
    r = oracle.rows(zb, zq)
    tr = otok.token_rows(zb, zq, t, r.lse_base, r.lse_quant)
    return tr.logp_base, tr.logp_quant, tr.dp, tr.state


def oracle_sum(lpb, lpq, dp, st):
    return otok.token_summary(otok.TokenRows(np.asarray(lpb, float), np.asarray(lpq, float),
                                             np.asarray(dp, float), np.asarray(st, np.uint8)))


@pytest.mark.parametrize("pin", pt.ROW_PINS, ids=lambda p: p.__name__)
def test_oracle_token_rows_satisfy_pin(pin):
    assert pin(oracle_tok)


@pytest.mark.parametrize("pin", pt.SUM_PINS, ids=lambda p: p.__name__)
def test_oracle_token_summary_satisfies_pin(pin):
    assert pin(oracle_sum)


# ---- mutants: plausible mistakes, each of which some pin must catch ----

def _lse(z):
    m = z.max(axis=1, keepdims=True)
    return (m + np.log(np.exp(z - m).sum(axis=1, keepdims=True)))[:, 0]


def _good_tok(zb, zq, t, *, swap_lse=False, flip_dp=False, shift_token=False, clamp_invalid=False):
    zb = np.atleast_2d(np.asarray(zb, float))
    zq = np.atleast_2d(np.asarray(zq, float))
    n, v = zb.shape
    t = np.asarray(t, np.int64)
    st = np.where(t < 0, 0, np.where(t >= v, 2, 1)).astype(np.uint8)
    if clamp_invalid:
        st[t >= v] = 1
    lb, lq = _lse(zb), _lse(zq)
    if swap_lse:
        lb, lq = lq, lb
    lpb = np.full(n, np.nan)
    lpq = np.full(n, np.nan)
    for r in range(n):
        if st[r] != 1:
            continue
        i = min(int(t[r]), v - 1)
        if shift_token:
            i = min(i + 1, v - 1)
        lpb[r] = zb[r, i] - lb[r]
        lpq[r] = zq[r, i] - lq[r]
    dp = np.exp(lpq) - np.exp(lpb)
    if flip_dp:
        dp = -dp
    return lpb, lpq, dp, st


def _exp(x):
    return math.exp(x) if x < math.log(sys.float_info.max) else math.inf


def _good_sum(lpb, lpq, dp, st, *, arith_ppl=False, rms_no_sqrt=False, count_all=False, ratio_of_ppls=False):
    sel = st == 1
    n = int(sel.sum())
    den = len(st) if count_all else n

    class S:
        pass

    s = S()
    s.n_scored, s.n_invalid = n, int((st == 2).sum())
    if n == 0:
        s.ppl_base = s.ppl_quant = s.ppl_ratio = s.dp_mean = s.dp_rms = float("nan")
        return s
    b, q, d = lpb[sel], lpq[sel], dp[sel]
    if arith_ppl:
        s.ppl_base = float(np.mean(np.exp(-b)))
        s.ppl_quant = float(np.mean(np.exp(-q)))
    else:
        s.ppl_base = _exp(-math.fsum(b.tolist()) / den)
        s.ppl_quant = _exp(-math.fsum(q.tolist()) / den)
    if ratio_of_ppls:
        s.ppl_ratio = s.ppl_quant / s.ppl_base
    else:
        s.ppl_ratio = _exp(math.fsum((b - q).tolist()) / den)
    s.dp_mean = math.fsum(d.tolist()) / den
    ms = math.fsum((d * d).tolist()) / den
    s.dp_rms = ms if rms_no_sqrt else math.sqrt(ms)
    return s


ROW_MUTANTS = {
    "swapped_normalisers": dict(swap_lse=True),
    "dp_sign_flipped": dict(flip_dp=True),
    "next_index_gathered": dict(shift_token=True),
    "invalid_ids_clamped_and_scored": dict(clamp_invalid=True),
}
SUM_MUTANTS = {
    "arithmetic_mean_of_inverse_probabilities": dict(arith_ppl=True),
    "rms_without_root": dict(rms_no_sqrt=True),
    "means_over_all_rows": dict(count_all=True),
    "ratio_of_overflowed_perplexities": dict(ratio_of_ppls=True),
}


def test_mutant_harness_is_sound():
    for pin in pt.ROW_PINS:
        assert pin(_good_tok), pin.__name__
    for pin in pt.SUM_PINS:
        assert pin(_good_sum), pin.__name__


@pytest.mark.parametrize("name", list(ROW_MUTANTS))
def test_row_pins_reject_mutant(name):
    kw = ROW_MUTANTS[name]
    impl = lambda zb, zq, t: _good_tok(zb, zq, t, **kw)  # noqa: E731
    assert not all(pin(impl) for pin in pt.ROW_PINS)


@pytest.mark.parametrize("name", list(SUM_MUTANTS))
def test_summary_pins_reject_mutant(name):
    kw = SUM_MUTANTS[name]
    impl = lambda *a: _good_sum(*a, **kw)  # noqa: E731
    assert not all(pin(impl) for pin in pt.SUM_PINS)


def test_token_rows_on_bf16_bits_match_widened_values():
    g = np.random.default_rng(30)
    zb = g.normal(0, 4.0, (5, 96)).astype(np.float32)
    bits = (zb.view(np.uint32) >> 16).astype(np.uint16)           # truncation: any bf16 pattern will do
    wide = oracle.bf16_bits_to_f64(bits)
    t = g.integers(0, 96, 5)
    r1 = oracle.rows(bits, bits)
    r2 = oracle.rows(wide, wide)
    a = otok.token_rows(bits, bits, t, r1.lse_base, r1.lse_quant)
    b = otok.token_rows(wide, wide, t, r2.lse_base, r2.lse_quant)
    assert np.array_equal(a.logp_base, b.logp_base) and np.array_equal(a.dp, b.dp)
    assert np.all(a.dp == 0.0)
