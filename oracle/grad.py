"""Float64 reference for the gradient of the per-token KL divergence with
respect to the quantized model's logits (test infrastructure).

TEST INFRASTRUCTURE ONLY, like the rest of this package.

The GSQ-RCO model card ("How it was made", step 7) tunes the quantized
model's continuous values by minimising KL(BF16 || quantized) of the
next-token distributions; the backward pass of that loss starts from its
derivative with respect to the quantized logits. For one row, with
p = softmax(z_base) and q = softmax(z_quant),

    KL = sum_i p_i log p_i - sum_i p_i z_quant[i] + lse(z_quant),

and since d lse(z)/d z_i = softmax(z)_i the derivative is

    dKL / dz_quant[i] = q_i - p_i.

A loss that averages KL over rows scales it by the row weight, passed in as
``scale`` (1/N for the mean over N rows).

Here p_i = exp(z_base[i] - lse_base) and q_i = exp(z_quant[i] - lse_quant),
with the float64 log-normalisers from the C reference, and the difference is
taken in float64.
"""
from __future__ import annotations

import numpy as np


def _f64(a: np.ndarray) -> np.ndarray:
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


def grad_rows(base: np.ndarray, quant: np.ndarray, lse_base: np.ndarray, lse_quant: np.ndarray,
              scale: float = 1.0):
    """Return (g, p, q): float64 [n, vocab] arrays with g = scale * (q - p)."""
    zb = _f64(np.atleast_2d(base))
    zq = _f64(np.atleast_2d(quant))
    p = np.exp(zb - np.asarray(lse_base, np.float64)[:, None])
    q = np.exp(zq - np.asarray(lse_quant, np.float64)[:, None])
    return scale * (q - p), p, q
