"""The top-K + rest-of-mass oracle against its pins, and mutants the pins reject."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from oracle import topk as otk
from tests import pins_topk as pk


def oracle_c(zb, k):
    zb = np.atleast_2d(zb)
    return otk.compress(zb, k, oracle.rows(zb, zb).lse_base)


def oracle_kl(t, zq):
    zq = np.atleast_2d(zq)
    r = otk.kl_topk(t, zq, oracle.rows(zq, zq).lse_base)
    return r.kl, r.argmax_quant, r.match


@pytest.mark.parametrize("pin", pk.ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_topk_satisfies_pin(pin):
    assert pin(oracle_c, oracle_kl)


def test_storage_rounding_is_float32():
    g = np.random.default_rng(70)
    zb = g.normal(0, 3.0, (3, 400))
    t = otk.to_storage(oracle_c(zb, 32))
    assert t.idx.dtype == np.int32 and t.logp.dtype == np.float32 and t.rest.dtype == np.float32


# ---- mutants ----

def _lse(z):
    m = z.max(axis=1, keepdims=True)
    return (m + np.log(np.exp(z - m).sum(axis=1, keepdims=True)))[:, 0]


def _good_c(zb, k, *, highest_ties=False):
    zb = np.atleast_2d(np.asarray(zb, float))
    n, v = zb.shape
    lse = _lse(zb)
    idx = np.empty((n, k), np.int64)
    for r in range(n):
        if highest_ties:
            order = sorted(range(v), key=lambda i: (-zb[r, i], -i))[:k]
        else:
            order = sorted(range(v), key=lambda i: (-zb[r, i], i))[:k]
        idx[r] = order
    logp = np.take_along_axis(zb, idx, 1) - lse[:, None]
    rest = np.array([np.exp(np.delete(zb[r], idx[r]) - lse[r]).sum() for r in range(n)])
    return otk.TopK(idx, logp, rest)


def _good_kl(t, zq, *, drop_rest=False, renormalise=False, rest_from_base=False):
    zq = np.atleast_2d(np.asarray(zq, float))
    n, v = zq.shape
    lse = _lse(zq)
    kl = np.empty(n)
    for r in range(n):
        sel = np.asarray(t.idx[r])
        lp = np.asarray(t.logp[r], float)
        logq = zq[r, sel] - lse[r]
        if renormalise:                       # KL over the stored tokens only, both renormalised
            lp = lp - np.log(np.exp(lp).sum())
            logq = logq - np.log(np.exp(logq).sum())
        s = float(np.sum(np.exp(lp) * (lp - logq)))
        R = float(t.rest[r])
        Q = float(np.exp(np.delete(zq[r], sel) - lse[r]).sum()) if sel.size < v else 0.0
        if rest_from_base:
            Q = 1.0 - float(np.exp(lp).sum())
        if R > 0 and not drop_rest and not renormalise:
            s += R * (np.log(R) - np.log(Q))
        kl[r] = s
    am = np.argmax(zq, axis=1)
    return kl, am, (am == np.asarray(t.idx)[:, 0]).astype(np.uint8)


C_MUTANTS = {"highest_index_ties": dict(highest_ties=True)}
KL_MUTANTS = {"rest_term_dropped": dict(drop_rest=True), "renormalised_over_stored": dict(renormalise=True),
              "quant_rest_from_base": dict(rest_from_base=True)}


def test_mutant_harness_is_sound():
    for pin in pk.ALL_PINS:
        assert pin(_good_c, _good_kl), pin.__name__


@pytest.mark.parametrize("name", list(C_MUTANTS))
def test_pins_reject_compress_mutant(name):
    kw = C_MUTANTS[name]
    assert not all(pin(lambda zb, k: _good_c(zb, k, **kw), _good_kl) for pin in pk.ALL_PINS)


@pytest.mark.parametrize("name", list(KL_MUTANTS))
def test_pins_reject_divergence_mutant(name):
    kw = KL_MUTANTS[name]
    assert not all(pin(_good_c, lambda t, zq: _good_kl(t, zq, **kw)) for pin in pk.ALL_PINS)


# ---- gradient of KL_K ----

def oracle_g(t, zq, scale):
    zq = np.atleast_2d(zq)
    return otk.grad_topk(t, zq, oracle.rows(zq, zq).lse_base, scale)


@pytest.mark.parametrize("pin", pk.GRAD_PINS, ids=lambda p: p.__name__)
def test_oracle_topk_grad_satisfies_pin(pin):
    assert pin(oracle_c, oracle_g)


def _good_g(t, zq, scale, *, full_grad=False, rest_unscaled=False, flip=False):
    zq = np.atleast_2d(np.asarray(zq, float))
    n, v = zq.shape
    out = np.empty((n, v))
    for r in range(n):
        q = np.exp(zq[r] - zq[r].max())
        q /= q.sum()
        sel = np.asarray(t.idx[r])
        p = np.exp(np.asarray(t.logp[r], float))
        R = float(t.rest[r])
        other = np.ones(v, bool)
        other[sel] = False
        row = q.copy()
        if full_grad:                              # treats the rest as if spread like the base: ignores R / Q_rest
            row[sel] -= p
        else:
            row *= (p.sum() + R)
            if R > 0:
                row[other] -= (R if rest_unscaled else R * q[other] / q[other].sum())
            row[sel] -= p
        out[r] = -scale * row if flip else scale * row
    return out


G_MUTANTS = {"rest_ignored": dict(full_grad=True), "rest_not_proportional": dict(rest_unscaled=True),
             "sign_flipped": dict(flip=True)}


def test_topk_grad_mutant_harness_is_sound():
    for pin in pk.GRAD_PINS:
        assert pin(oracle_c, _good_g), pin.__name__


@pytest.mark.parametrize("name", list(G_MUTANTS))
def test_topk_grad_pins_reject_mutant(name):
    kw = G_MUTANTS[name]
    assert not all(pin(oracle_c, lambda t, zq, s: _good_g(t, zq, s, **kw)) for pin in pk.GRAD_PINS)
