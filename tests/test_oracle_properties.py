"""Randomized checks of the oracle (no GPU): rows drawn by hypothesis
(derandomized, so every run draws the same cases) against 50-digit decimal
arithmetic and against the invariants the definitions fix. The drawn rows mix
repeated values (ties, +0 and -0), offsets up to +-90 nats, identical,
shifted, perturbed and permuted quant rows."""
from decimal import Decimal, localcontext

import numpy as np
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle
from oracle import grad as ograd
from oracle import tokens as otok
from oracle import topk as otk
from oracle.bruteforce import bruteforce

EPS = np.finfo(np.float64).eps
SETTINGS = settings(max_examples=150, deadline=None, derandomize=True, database=None,
                    suppress_health_check=[HealthCheck.too_slow, HealthCheck.data_too_large])
VALUES = st.one_of(st.floats(min_value=-90.0, max_value=90.0, allow_nan=False, width=32),
                   st.sampled_from([0.0, -0.0, 1.0, 2.5, -7.0]))


@st.composite
def row_pairs(draw, max_v=10):
    v = draw(st.integers(1, max_v))
    zb = np.array(draw(st.lists(VALUES, min_size=v, max_size=v)), np.float64)
    mode = draw(st.sampled_from(["independent", "identical", "shifted", "perturbed", "permuted"]))
    if mode == "independent":
        zq = np.array(draw(st.lists(VALUES, min_size=v, max_size=v)), np.float64)
    elif mode == "identical":
        zq = zb.copy()
    elif mode == "shifted":
        zq = zb + draw(st.floats(min_value=-50.0, max_value=50.0, width=32))
    elif mode == "perturbed":
        eps = draw(st.sampled_from([1e-6, 1e-3, 0.1, 1.0]))
        zq = zb + eps * np.array(draw(st.lists(st.floats(-1.0, 1.0, width=32), min_size=v, max_size=v)))
    else:
        zq = zb[np.array(draw(st.permutations(list(range(v)))), np.int64)]
    return zb, zq


def _floor(zb, zq):
    return 16 * EPS * (1.0 + max(np.abs(zb).max(), np.abs(zq).max()))


def _rows(zb, zq):
    return oracle.rows(np.ascontiguousarray(zb[None], np.float64), np.ascontiguousarray(zq[None], np.float64))


def _dec_logsoftmax(z):
    with localcontext() as ctx:
        ctx.prec = 50
        e = [Decimal(float(x)).exp() for x in z]
        s = sum(e, Decimal(0))
        return [Decimal(float(x)) - s.ln() for x in z]


@SETTINGS
@given(row_pairs())
def test_kl_and_argmaxes_match_50_digit_arithmetic(pair):
    zb, zq = pair
    o = _rows(zb, zq)
    kl, ib, iq = bruteforce(zb, zq)
    assert abs(o.kl[0] - float(kl)) <= max(1e-12 * abs(float(kl)), _floor(zb, zq))
    assert int(o.argmax_base[0]) == ib and int(o.argmax_quant[0]) == iq
    assert bool(o.match[0]) == (ib == iq)


@SETTINGS
@given(row_pairs(), st.floats(-80.0, 80.0, width=32), st.floats(-80.0, 80.0, width=32))
def test_kl_invariants(pair, a, b):
    zb, zq = pair
    o = _rows(zb, zq)
    fl = _floor(zb, zq) + 16 * EPS * (abs(a) + abs(b))
    assert o.kl[0] >= -fl                                                  # Gibbs
    assert _rows(zb, zb).kl[0] == 0.0                                      # KL(p || p) = 0 exactly
    s = _rows(zb + a, zq + b)                                              # constants cancel in softmax
    assert abs(s.kl[0] - o.kl[0]) <= max(1e-12 * abs(o.kl[0]), fl)
    perm = np.arange(zb.size)[::-1]
    p = _rows(zb[perm], zq[perm])                                          # joint relabelling
    assert abs(p.kl[0] - o.kl[0]) <= max(1e-12 * abs(o.kl[0]), fl)


@SETTINGS
@given(row_pairs(), st.data())
def test_topk_stored_form_and_coarsened_kl(pair, data):
    zb, zq = pair
    v = zb.size
    k = data.draw(st.integers(1, v))
    full = _rows(zb, zq)
    lse_b = _rows(zb, zb).lse_base
    t = otk.compress(zb[None], k, lse_b)
    # the stored tokens: the k largest values, equal values by lowest index, in that order
    order = sorted(range(v), key=lambda i: (-float(zb[i]) if zb[i] != 0 else 0.0, i))
    assert [int(i) for i in t.idx[0]] == order[:k]
    lp = _dec_logsoftmax(zb)
    for j, i in enumerate(order[:k]):
        assert abs(t.logp[0, j] - float(lp[i])) <= _floor(zb, zb)
    with localcontext() as ctx:
        ctx.prec = 50
        rest = sum((lp[i].exp() for i in order[k:]), Decimal(0))
    assert abs(t.rest[0] - float(rest)) <= 1e-12 * float(rest) + 1e-300
    lse_q = _rows(zq, zq).lse_base
    r = otk.kl_topk(t, zq[None], lse_q)
    fl = _floor(zb, zq)
    assert r.kl[0] <= full.kl[0] + max(1e-12 * abs(full.kl[0]), fl)      # coarsening never adds divergence
    assert r.kl[0] >= -fl
    if k == v:
        assert abs(r.kl[0] - full.kl[0]) <= max(1e-12 * abs(full.kl[0]), fl)


@SETTINGS
@given(row_pairs(), st.data())
def test_next_token_log_probabilities(pair, data):
    zb, zq = pair
    v = zb.size
    t = data.draw(st.integers(0, v - 1))
    o = _rows(zb, zq)
    tr = otok.token_rows(zb[None], zq[None], np.array([t], np.int64), o.lse_base, o.lse_quant)
    lb, lq = _dec_logsoftmax(zb)[t], _dec_logsoftmax(zq)[t]
    assert abs(tr.logp_base[0] - float(lb)) <= _floor(zb, zq)
    assert abs(tr.logp_quant[0] - float(lq)) <= _floor(zb, zq)
    with localcontext() as ctx:
        ctx.prec = 50
        dp = lq.exp() - lb.exp()
    assert abs(tr.dp[0] - float(dp)) <= _floor(zb, zq)


@SETTINGS
@given(row_pairs(), st.floats(-4.0, 4.0, width=32))
def test_gradient_rows(pair, scale):
    zb, zq = pair
    o = _rows(zb, zq)
    g, p, q = ograd.grad_rows(zb[None], zq[None], o.lse_base, o.lse_quant, scale)
    lb, lq = _dec_logsoftmax(zb), _dec_logsoftmax(zq)
    with localcontext() as ctx:
        ctx.prec = 50
        want = [Decimal(float(scale)) * (q_.exp() - b.exp()) for b, q_ in zip(lb, lq)]
    fl = _floor(zb, zq) * max(abs(scale), 1.0)
    assert np.all(np.abs(g[0] - np.array([float(w) for w in want])) <= fl)
    assert abs(g[0].sum()) <= fl * zb.size                                 # a softmax difference sums to 0
