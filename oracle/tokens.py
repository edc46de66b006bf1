"""Float64 reference for the token-conditioned metrics (test infrastructure).

TEST INFRASTRUCTURE ONLY, like the rest of this package.

Each row is one position of a text; ``tokens[r]`` is the token that actually
follows it. With ``lse`` the log-normaliser of a row (from the C reference):

* ``logp_base = z_base[t] - lse_base`` and ``logp_quant = z_quant[t] -
  lse_quant``: the log-probability each model gives the actual next token;
* ``dp = exp(logp_quant) - exp(logp_base)``: how much probability the
  quantized model gains (or loses) on that token.

Summaries over the scored rows (token id in ``[0, vocab)``):

* ``ppl = exp(-mean logp)`` for each model. The "Raw benchmark data" table of
  the "Qwen3.6 27B Quantization Benchmark" page reports it for the quantized
  model as "Mean PPL(Q)";
* ``ppl_ratio = ppl_quant / ppl_base``: the perplexity ratio of the GSQ-RCO
  model card's "Quality" section;
* ``dp_mean``: the average change of the correct token's probability, the
  "points" the same section quotes;
* ``dp_rms = sqrt(mean dp^2)``: the "RMS Δp (%)" column of the Qwen3.6 table
  (as a fraction here, not in percent).

The pages name these quantities without writing them out; the formulas above
are the plainest reading of the names (perplexity is the exponential of the
mean negative log-likelihood; Δp is the quantized model's probability of the
token minus the base model's).

Row states: 1 = scored, 0 = not scored (negative id: a position with no next
token, such as the last of a context), 2 = invalid (id >= vocab, not scored).
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

NOT_SCORED, SCORED, INVALID = 0, 1, 2


@dataclass
class TokenRows:
    logp_base: np.ndarray   # float64 [n], NaN where not scored
    logp_quant: np.ndarray  # float64 [n], NaN where not scored
    dp: np.ndarray          # float64 [n], NaN where not scored
    state: np.ndarray       # uint8 [n]


@dataclass
class TokenSummary:
    n_scored: int
    n_invalid: int
    logp_base_sum: float
    logp_quant_sum: float
    ppl_base: float
    ppl_quant: float
    ppl_ratio: float
    dp_mean: float
    dp_rms: float


def _f64(a: np.ndarray) -> np.ndarray:
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


def token_rows(base: np.ndarray, quant: np.ndarray, tokens: np.ndarray,
               lse_base: np.ndarray, lse_quant: np.ndarray) -> TokenRows:
    """Per-row log-probabilities of the next token and their probability change.

    ``base``/``quant`` are [n, vocab] (float32, float64 or raw bfloat16 bits),
    ``tokens`` int [n], ``lse_*`` the float64 log-normalisers of each row.
    """
    base = np.atleast_2d(base)
    quant = np.atleast_2d(quant)
    n, v = base.shape
    tokens = np.asarray(tokens, dtype=np.int64).reshape(n)
    state = np.where(tokens < 0, NOT_SCORED, np.where(tokens >= v, INVALID, SCORED)).astype(np.uint8)
    lpb = np.full(n, np.nan)
    lpq = np.full(n, np.nan)
    dp = np.full(n, np.nan)
    for r in range(n):
        if state[r] != SCORED:
            continue
        t = int(tokens[r])
        zb = float(_f64(base[r, t:t + 1])[0])
        zq = float(_f64(quant[r, t:t + 1])[0])
        lpb[r] = zb - float(lse_base[r])
        lpq[r] = zq - float(lse_quant[r])
        dp[r] = math.exp(lpq[r]) - math.exp(lpb[r])
    return TokenRows(lpb, lpq, dp, state)


def _exp(x: float) -> float:
    """exp in float64, +inf past the largest double (where math.exp raises)."""
    try:
        return math.exp(x)
    except OverflowError:
        return math.inf


def token_summary(tr: TokenRows) -> TokenSummary:
    """Perplexities, their ratio, mean and RMS of dp over the scored rows, with
    exactly rounded sums (math.fsum). Means over zero scored rows are NaN. A
    perplexity past the largest double is +inf; the ratio ppl_quant / ppl_base
    is formed as the one exponential exp((sum log p_base - sum log p_quant) / n),
    the same quantity, so it stays finite where both perplexities overflow."""
    sel = tr.state == SCORED
    n = int(np.count_nonzero(sel))
    n_bad = int(np.count_nonzero(tr.state == INVALID))
    sb = math.fsum(tr.logp_base[sel].tolist())
    sq = math.fsum(tr.logp_quant[sel].tolist())
    if n == 0:
        nan = float("nan")
        return TokenSummary(0, n_bad, sb, sq, nan, nan, nan, nan, nan)
    ppl_b = _exp(-sb / n)
    ppl_q = _exp(-sq / n)
    ratio = _exp((sb - sq) / n)
    d = tr.dp[sel].tolist()
    dp_mean = math.fsum(d) / n
    dp_rms = math.sqrt(math.fsum(x * x for x in d) / n)
    return TokenSummary(n, n_bad, sb, sq, ppl_b, ppl_q, ratio, dp_mean, dp_rms)
