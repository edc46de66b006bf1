"""The gradient oracle against its pins, and mutants that the pins reject."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from oracle import grad as ograd
from tests import pins_grad as pg


def oracle_grad(zb, zq, scale):
    zb = np.atleast_2d(zb)
    zq = np.atleast_2d(zq)
    r = oracle.rows(zb, zq)
    return ograd.grad_rows(zb, zq, r.lse_base, r.lse_quant, scale)[0]


@pytest.mark.parametrize("pin", pg.ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_grad_satisfies_pin(pin):
    assert pin(oracle_grad)


def _softmax(z):
    e = np.exp(z - z.max(axis=1, keepdims=True))
    return e / e.sum(axis=1, keepdims=True)


def _good(zb, zq, scale, *, flip=False, unnormalised=False, logdiff=False, base_grad=False, no_scale=False):
    zb = np.atleast_2d(np.asarray(zb, float))
    zq = np.atleast_2d(np.asarray(zq, float))
    p, q = _softmax(zb), _softmax(zq)
    if unnormalised:
        m = np.maximum(zb.max(axis=1, keepdims=True), zq.max(axis=1, keepdims=True))
        p, q = np.exp(zb - m), np.exp(zq - m)
    if logdiff:
        g = np.log(q) - np.log(p)
    elif base_grad:                                   # derivative in the base logits instead
        kl = np.sum(p * (np.log(p) - np.log(q)), axis=1, keepdims=True)
        g = p * (np.log(p) - np.log(q) - kl)
    else:
        g = q - p
    if flip:
        g = -g
    return g if no_scale else scale * g


MUTANTS = {
    "sign_flipped": dict(flip=True),
    "unnormalised": dict(unnormalised=True),
    "log_difference": dict(logdiff=True),
    "base_logit_gradient": dict(base_grad=True),
    "row_weight_ignored": dict(no_scale=True),
}


def test_mutant_harness_is_sound():
    for pin in pg.ALL_PINS:
        assert pin(_good), pin.__name__


@pytest.mark.parametrize("name", list(MUTANTS))
def test_pins_reject_mutant(name):
    kw = MUTANTS[name]
    impl = lambda zb, zq, s: _good(zb, zq, s, **kw)  # noqa: E731
    assert not all(pin(impl) for pin in pg.ALL_PINS)
