"""Float64 reference for base rows stored as their top-K tokens plus the rest
of the mass, and for the divergence of a full quantized row from such a row
(test infrastructure).

TEST INFRASTRUCTURE ONLY, like the rest of this package.

The GSQ-RCO model card ("How it was made", step 7) tunes against "the top-128
distributions (and the rest of the mass)" of the BF16 model: per position,
the K most probable tokens with their probabilities, and the total
probability of all other tokens. The card does not write out the divergence
used against that form. The reading taken here is the plainest one: both
distributions are coarsened to the same K + 1 outcomes -- the K stored tokens
and one outcome "any other token" -- and the divergence is the ordinary KL of
the coarsened distributions,

    KL_K = sum_k p_k (log p_k - log q_k) + R (log R - log Q_rest),

with p_k, R the stored base probabilities and rest mass, q_k the quantized
model's probabilities of the same tokens and Q_rest the quantized model's mass
outside them (a term with R = 0 is 0). It equals the full KL when K = V and,
being a coarsening, never exceeds it.

Which tokens are "top": the K largest base logits, equal logits ordered by
lowest index (the same tie rule as the argmax), listed in that order, so the
first stored token is the base argmax. Stored form per row: ``idx`` (int), K
log-probabilities ``logp = z[idx] - lse`` and the rest mass
``rest = sum of exp(z_i - lse) over the other tokens``, summed directly (never
as 1 minus the stored mass).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


def _f64(a: np.ndarray) -> np.ndarray:
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


@dataclass
class TopK:
    idx: np.ndarray   # int64 [n, K], most probable first, ties by lowest index
    logp: np.ndarray  # [n, K] log-probabilities of those tokens
    rest: np.ndarray  # [n] probability mass of every other token


def select(z: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest entries of a float64 row, largest first, equal
    values by lowest index (a stable sort of the negated values)."""
    return np.argsort(-z, kind="stable")[:k]


def compress(base: np.ndarray, k: int, lse_base: np.ndarray) -> TopK:
    """Stored form of every row of ``base`` ([n, V]); lse_base from the C reference."""
    zb = _f64(np.atleast_2d(base))
    n, v = zb.shape
    if not 1 <= k <= v:
        raise ValueError("need 1 <= k <= vocab")
    idx = np.empty((n, k), np.int64)
    logp = np.empty((n, k))
    rest = np.empty(n)
    for r in range(n):
        sel = select(zb[r], k)
        other = np.ones(v, bool)
        other[sel] = False
        idx[r] = sel
        logp[r] = zb[r, sel] - lse_base[r]
        rest[r] = float(np.sum(np.exp(zb[r, other] - lse_base[r])))
    return TopK(idx, logp, rest)


def to_storage(t: TopK) -> TopK:
    """The stored form as the library keeps it: int32 indices, float32 values."""
    return TopK(t.idx.astype(np.int32), t.logp.astype(np.float32), t.rest.astype(np.float32))


@dataclass
class TopKResult:
    kl: np.ndarray            # float64 [n]
    argmax_quant: np.ndarray  # int64 [n], lowest index of the quant row's maximum
    match: np.ndarray         # uint8 [n], argmax_quant == idx[:, 0]
    q_rest: np.ndarray        # float64 [n], quantized mass outside the stored tokens


def kl_topk(t: TopK, quant: np.ndarray, lse_quant: np.ndarray) -> TopKResult:
    """KL of the coarsened distributions for each row; lse_quant from the C
    reference. The stored values are used exactly as given (widened to float64)."""
    zq = _f64(np.atleast_2d(quant))
    n, v = zq.shape
    kl = np.empty(n)
    qrest = np.empty(n)
    for r in range(n):
        sel = np.asarray(t.idx[r], np.int64)
        lp = np.asarray(t.logp[r], np.float64)
        other = np.ones(v, bool)
        other[sel] = False
        logq = zq[r, sel] - lse_quant[r]
        qr = float(np.sum(np.exp(zq[r, other] - lse_quant[r])))
        R = float(t.rest[r])
        s = float(np.sum(np.exp(lp) * (lp - logq)))
        if R > 0.0:
            s += R * (np.log(R) - np.log(qr))
        kl[r] = s
        qrest[r] = qr
    am = np.argmax(zq, axis=1).astype(np.int64)
    match = (am == np.asarray(t.idx[:, 0], np.int64)).astype(np.uint8)
    return TopKResult(kl, am, match, qrest)


def grad_topk(t: TopK, quant: np.ndarray, lse_quant: np.ndarray, scale: float = 1.0) -> np.ndarray:
    """Gradient of KL_K with respect to the quantized logits, times ``scale``
    (the row's weight in a loss), for the stored values as given (float64).

    With q = softmax(z_quant), S the stored tokens, P = sum_k p_k, R the rest
    mass and Q_rest = sum of q_i over the other tokens, differentiating
    KL_K = sum_k p_k (log p_k - log q_k) + R (log R - log Q_rest) through
    d log q_k / d z_j = [j = k] - q_j and
    d log Q_rest / d z_j = [j not in S] q_j / Q_rest - q_j gives

        dKL_K / dz_j = q_j (P + R) - [j in S] p_j - [j not in S] R q_j / Q_rest

    (q - p for the full distribution when every token is stored). This is the
    derivative the model card's end-to-end tuning follows in its phase against
    the top-128 distributions ("How it was made" step 7).
    """
    zq = _f64(np.atleast_2d(quant))
    n, v = zq.shape
    g = np.empty((n, v))
    for r in range(n):
        q = np.exp(zq[r] - lse_quant[r])
        sel = np.asarray(t.idx[r], np.int64)
        p = np.exp(np.asarray(t.logp[r], np.float64))
        R = float(t.rest[r])
        other = np.ones(v, bool)
        other[sel] = False
        Q = float(np.sum(q[other]))
        row = q * (float(np.sum(p)) + R)
        if R > 0.0:
            row[other] -= R * q[other] / Q
        row[sel] -= p
        g[r] = scale * row
    return g
