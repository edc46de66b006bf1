"""The oracle checked against what the definition fixes (no GPU).

Both oracle implementations (the C reference and the SciPy twin) must satisfy
every pin in tests/pins.py. Broken variants of the definition -- reversed
divergence direction, a dropped normaliser, base-2 logs, the wrong tie rule, a
transposed weighting -- are planted on the CPU and must each fail at least one
pin, which shows that the pins would catch such a mistake in the oracle.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from tests import pins


def c_impl(zb, zq):
    r = oracle.rows(np.ascontiguousarray(zb, np.float64), np.ascontiguousarray(zq, np.float64))
    return r.kl, r.argmax_base, r.argmax_quant


def scipy_impl(zb, zq):
    kl, ib, iq, _ = oracle.rows_scipy(zb, zq)
    return kl, ib, iq


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
@pytest.mark.parametrize("impl", [c_impl, scipy_impl], ids=["c", "scipy"])
def test_oracle_satisfies_pin(impl, pin):
    assert pin(impl)


# ---------------------------------------------------------------- mutants ---

def _lse(z):
    m = z.max(axis=1, keepdims=True)
    return (m + np.log(np.exp(z - m).sum(axis=1, keepdims=True)))


def _good(zb, zq):
    lb, lq = _lse(zb), _lse(zq)
    p = np.exp(zb - lb)
    kl = np.sum(p * ((zb - lb) - (zq - lq)), axis=1)
    return kl, np.argmax(zb, 1), np.argmax(zq, 1)


def mut_reversed_direction(zb, zq):          # KL(Q || P)
    kl, ib, iq = _good(zq, zb)
    return kl, np.argmax(zb, 1), np.argmax(zq, 1)


def mut_dropped_quant_normaliser(zb, zq):     # log q taken as raw logits
    lb = _lse(zb)
    p = np.exp(zb - lb)
    return np.sum(p * ((zb - lb) - zq), axis=1), np.argmax(zb, 1), np.argmax(zq, 1)


def mut_log2(zb, zq):                         # bits instead of nats
    kl, ib, iq = _good(zb, zq)
    return kl / math.log(2.0), ib, iq


def mut_highest_index_ties(zb, zq):
    kl, _, _ = _good(zb, zq)
    v = zb.shape[1]
    return kl, v - 1 - np.argmax(zb[:, ::-1], 1), v - 1 - np.argmax(zq[:, ::-1], 1)


def mut_quant_weights(zb, zq):                # weights from q instead of p
    lb, lq = _lse(zb), _lse(zq)
    q = np.exp(zq - lq)
    return np.sum(q * ((zb - lb) - (zq - lq)), axis=1), np.argmax(zb, 1), np.argmax(zq, 1)


def mut_missing_max_shift_sign(zb, zq):       # lse with the shift subtracted twice
    m = zb.max(axis=1, keepdims=True)
    lb = np.log(np.exp(zb - m).sum(axis=1, keepdims=True))   # forgot "+ m"
    lq = _lse(zq)
    p = np.exp(zb - lb - m)
    return np.sum(p * ((zb - lb) - (zq - lq)), axis=1), np.argmax(zb, 1), np.argmax(zq, 1)


def mut_off_by_one_argmax(zb, zq):
    kl, ib, iq = _good(zb, zq)
    return kl, np.minimum(ib + (ib % 7 == 3), zb.shape[1] - 1), iq


MUTANTS = [mut_reversed_direction, mut_dropped_quant_normaliser, mut_log2,
           mut_highest_index_ties, mut_quant_weights, mut_missing_max_shift_sign,
           mut_off_by_one_argmax]


def test_reference_mutant_harness_is_sound():
    # the unbroken NumPy formula passes every pin, so failures below are the mutations'
    for pin in pins.ALL_PINS:
        assert pin(_good), pin.__name__


@pytest.mark.parametrize("mutant", MUTANTS, ids=lambda m: m.__name__)
def test_pins_reject_mutant(mutant):
    with np.errstate(all="ignore"):
        failed = [p.__name__ for p in pins.ALL_PINS if not p(mutant)]
    assert failed, f"{mutant.__name__} passed every pin"


# ----------------------------------------------------------- oracle details ---

def test_c_oracle_matches_scipy_twin_on_config_shaped_rows():
    """The C reference and the SciPy twin agree on rows of every config's recipe."""
    import synth
    for name in ["c1", "c2", "c3", "c4", "c5"]:
        cfg = synth.CONFIGS[name].scaled(n_rows=4, vocab=4096)
        b, q = synth.generate(cfg)
        nb, nq = synth.to_numpy_bits(b), synth.to_numpy_bits(q)
        r = oracle.rows(nb, nq)
        kl, ib, iq, m = oracle.rows_scipy(nb, nq)
        zb, zq = oracle.to_f64(nb), oracle.to_f64(nq)
        floor = pins._f64_floor(zb, zq)
        assert np.all(np.abs(r.kl - kl) <= np.maximum(1e-10 * np.abs(kl), floor)), name
        assert np.array_equal(r.argmax_base, ib) and np.array_equal(r.argmax_quant, iq)
        assert np.array_equal(r.match, m)


def test_bf16_and_f32_inputs_widen_exactly():
    g = np.random.default_rng(0)
    x = g.normal(0, 5, (3, 64)).astype(np.float32)
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)       # truncation: exact bf16 values
    as_f32 = (bits.astype(np.uint32) << 16).view(np.float32)
    r1 = oracle.rows(bits, bits[:, ::-1].copy())
    r2 = oracle.rows(as_f32, as_f32[:, ::-1].copy())
    r3 = oracle.rows(as_f32.astype(np.float64), as_f32[:, ::-1].astype(np.float64))
    assert np.array_equal(r1.kl, r2.kl) and np.array_equal(r2.kl, r3.kl)
    assert np.array_equal(r1.argmax_base, r3.argmax_base)


def test_lse_values():
    g = np.random.default_rng(1)
    z = g.normal(0, 3, (4, 333))
    r = oracle.rows(z, z + 1.0)
    ref = np.log(np.exp(z).sum(axis=1))
    assert np.allclose(r.lse_base, ref, rtol=1e-14)
    assert np.allclose(r.lse_quant, ref + 1.0, rtol=1e-14)


def test_single_token_vocabulary():
    r = oracle.rows(np.array([[3.0], [-1.0]]), np.array([[7.0], [2.0]]))
    assert np.all(r.kl == 0.0) and np.all(r.match == 1)
    assert np.all(r.argmax_base == 0) and np.all(r.argmax_quant == 0)


def test_zero_rows():
    r = oracle.rows(np.zeros((0, 5)), np.zeros((0, 5)))
    assert r.kl.shape == (0,)


def test_summary_exact_mean_and_lowest_row_max():
    kl = np.array([0.5, 2.0, 1e-17, 2.0, -1e-18] + [1e-3] * 1000)
    match = np.array([1, 0, 1, 1, 0] + [1] * 1000, np.uint8)
    s = oracle.summary(kl, match)
    from fractions import Fraction
    exact = sum(Fraction(float(v)) for v in kl) / len(kl)
    assert abs(Fraction(s.kld_mean) - exact) <= abs(exact) * Fraction(1, 10**15)
    assert s.kld_max == 2.0 and s.kld_max_row == 1
    assert s.n_match == 1003 and s.n_rows == 1005
    assert s.same_top1 == 1003 / 1005


def test_summary_rejects_empty():
    with pytest.raises(ValueError):
        oracle.summary(np.zeros(0), np.zeros(0, np.uint8))


# ------------------------------------------------------------ golden files ---

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "tiny_rows.json")


def test_golden_tiny_rows():
    with open(GOLDEN) as f:
        doc = json.load(f)
    assert doc["cases"], "empty golden file"
    for case in doc["cases"]:
        zb = np.array(case["base"], np.float64)
        zq = np.array(case["quant"], np.float64)
        r = oracle.rows(zb[None], zq[None])
        ref = float(case["kl"])
        assert abs(r.kl[0] - ref) <= max(1e-12 * abs(ref), 1e-15), case["name"]
        assert int(r.argmax_base[0]) == case["argmax_base"], case["name"]
        assert int(r.argmax_quant[0]) == case["argmax_quant"], case["name"]
        assert int(r.match[0]) == case["match"], case["name"]
