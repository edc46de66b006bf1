"""NumPy/SciPy float64 twin of the C oracle (test infrastructure).

A second, independently written evaluation of the same definition, assembled
from library primitives instead of hand-written loops: ``scipy.special``'s
``log_softmax``/``softmax`` give log p, p and q, ``rel_entr(p, q)`` gives the
elementwise ``p log(p/q)`` terms, and NumPy's ``argmax`` (documented to return
the first occurrence) gives the lowest-index argmax. Used to cross-check the C
reference; it shares no code with it.
"""
from __future__ import annotations

import numpy as np
from scipy import special


def _to_f64(arr: np.ndarray) -> np.ndarray:
    if arr.dtype == np.uint16:
        return (arr.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return np.asarray(arr, dtype=np.float64)


def rows_scipy(base: np.ndarray, quant: np.ndarray):
    """Return (kl[n], argmax_base[n], argmax_quant[n], match[n]) in float64/int64."""
    zb = _to_f64(np.atleast_2d(base))
    zq = _to_f64(np.atleast_2d(quant))
    p = special.softmax(zb, axis=1)
    q = special.softmax(zq, axis=1)
    kl = special.rel_entr(p, q).sum(axis=1)
    ib = np.argmax(zb, axis=1).astype(np.int64)
    iq = np.argmax(zq, axis=1).astype(np.int64)
    return kl, ib, iq, (ib == iq).astype(np.uint8)
