"""50-significant-digit brute force for tiny vocabularies (test infrastructure).

Every float input is converted to ``decimal.Decimal`` exactly, then
``p_i = e^{zb_i} / sum_j e^{zb_j}``, ``q_i`` likewise, and
``KL = sum_i p_i (ln p_i - ln q_i)`` -- the divergence of the quantized
distribution from the base one (base first), in nats, as the GSQ-RCO model
card's "How it was made" step 5 states it. No max-shift, no log-sum-exp: the
naive textbook formula, made safe by the working precision. Meant for
vocabularies of at most a few dozen entries.
"""
from __future__ import annotations

from decimal import Decimal, localcontext

import numpy as np


def _dec(x) -> Decimal:
    return Decimal(float(x))


def bruteforce(zb, zq, digits: int = 50):
    """Return (kl: Decimal, argmax_base: int, argmax_quant: int) for one row."""
    zb = [float(v) for v in np.asarray(zb, dtype=np.float64).ravel()]
    zq = [float(v) for v in np.asarray(zq, dtype=np.float64).ravel()]
    if len(zb) != len(zq) or not zb:
        raise ValueError("rows must be non-empty and of equal length")
    with localcontext() as ctx:
        ctx.prec = digits
        eb = [_dec(v).exp() for v in zb]
        eq = [_dec(v).exp() for v in zq]
        sb = sum(eb, Decimal(0))
        sq = sum(eq, Decimal(0))
        kl = Decimal(0)
        for b, q in zip(eb, eq):
            p_i = b / sb
            q_i = q / sq
            kl += p_i * (p_i.ln() - q_i.ln())
    # lowest index attaining the maximum, by explicit scan
    ib = 0
    for i, v in enumerate(zb):
        if v > zb[ib]:
            ib = i
    iq = 0
    for i, v in enumerate(zq):
        if v > zq[iq]:
            iq = i
    return kl, ib, iq
