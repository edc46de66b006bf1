"""Float64 CPU oracle for the quantized-vs-BF16 logit comparison.

TEST INFRASTRUCTURE ONLY. The test suite, the package smoke check and the
benchmark's CPU-baseline leg are the only code allowed to import this package.
It shares nothing with the HIP path (no kernels, headers, helpers or tables);
the two meet only through the seeded input bytes.

Three independent evaluations of the same definition live here (and, built
on the C reference's log-normalisers, ``tokens.py`` for the token-conditioned
metrics, ``grad.py`` for the gradient with respect to the quantized logits and
``topk.py`` for base rows stored as their top-K tokens plus the rest of the mass):

* ``rows``           -- the plain C reference (``kld_oracle.c``), float64,
                         OpenMP over rows; this is the parity oracle.
* ``rows_scipy``     -- a NumPy/SciPy float64 twin built from library
                         primitives (``scipy.special.softmax`` and ``rel_entr``).
* ``bruteforce``     -- 50-digit ``decimal`` arithmetic for tiny vocabularies.

Definition (see ``kld_oracle.c`` for the page citations): with
``p = softmax(z_base)`` and ``q = softmax(z_quant)`` at temperature 1,
``KL = sum_i p_i (log p_i - log q_i)`` in nats, the argmax of each row is the
lowest index attaining the maximum, and ``match`` is argmax equality.
Summaries: mean KLD over every row passed in, max KLD with the lowest row
index attaining it, and the number / fraction of matching rows.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass

import numpy as np

from .build import build_oracle, oracle_library_path

F32, BF16, F64 = 0, 1, 2

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    path = oracle_library_path()
    if not os.path.exists(path):
        build_oracle()
    _lib = open_library(path)
    return _lib


def open_library(path: str):
    """The C reference from a given build of kld_oracle.c (the in-tree one,
    or a copy compiled with other flags), ready for ``rows(..., lib=)``."""
    lib = ctypes.CDLL(path)
    i64 = ctypes.c_int64
    vp = ctypes.c_void_p
    lib.kldo_rows.argtypes = [vp, ctypes.c_int, vp, ctypes.c_int, i64, i64,
                              vp, vp, vp, vp, vp, vp, ctypes.c_int]
    lib.kldo_rows.restype = ctypes.c_int
    lib.kldo_max_threads.argtypes = [ctypes.c_int]
    lib.kldo_max_threads.restype = ctypes.c_int
    return lib


def dtype_code(arr: np.ndarray) -> int:
    """float32 -> F32, uint16 (raw bfloat16 bit patterns) -> BF16, float64 -> F64."""
    if arr.dtype == np.float32:
        return F32
    if arr.dtype == np.uint16:
        return BF16
    if arr.dtype == np.float64:
        return F64
    raise TypeError(f"unsupported oracle input dtype {arr.dtype}")


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of raw bfloat16 bit patterns (uint16) to float64."""
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def to_f64(arr: np.ndarray) -> np.ndarray:
    if arr.dtype == np.uint16:
        return bf16_bits_to_f64(arr)
    return arr.astype(np.float64)


@dataclass
class RowResults:
    kl: np.ndarray          # float64 [n]
    argmax_base: np.ndarray  # int64 [n]
    argmax_quant: np.ndarray  # int64 [n]
    match: np.ndarray       # uint8 [n]
    lse_base: np.ndarray    # float64 [n]
    lse_quant: np.ndarray   # float64 [n]


def rows(base: np.ndarray, quant: np.ndarray, n_threads: int = 0, lib=None) -> RowResults:
    """Evaluate every row of two [n_rows, vocab] arrays with the C reference
    (``lib``: another build of it, from ``open_library``)."""
    lib = lib or _load()
    if base.ndim == 1:
        base = base[None, :]
    if quant.ndim == 1:
        quant = quant[None, :]
    if base.shape != quant.shape:
        raise ValueError(f"shape mismatch {base.shape} vs {quant.shape}")
    base = np.ascontiguousarray(base)
    quant = np.ascontiguousarray(quant)
    n, v = base.shape
    out = RowResults(
        kl=np.empty(n, np.float64),
        argmax_base=np.empty(n, np.int64),
        argmax_quant=np.empty(n, np.int64),
        match=np.empty(n, np.uint8),
        lse_base=np.empty(n, np.float64),
        lse_quant=np.empty(n, np.float64),
    )
    if n == 0:
        return out
    st = lib.kldo_rows(base.ctypes.data, dtype_code(base), quant.ctypes.data,
                       dtype_code(quant), n, v,
                       out.kl.ctypes.data, out.argmax_base.ctypes.data,
                       out.argmax_quant.ctypes.data, out.match.ctypes.data,
                       out.lse_base.ctypes.data, out.lse_quant.ctypes.data,
                       int(n_threads))
    if st != 0:
        raise RuntimeError(f"kldo_rows failed with status {st}")
    return out


def max_threads(n_threads: int = 0, lib=None) -> int:
    return int((lib or _load()).kldo_max_threads(int(n_threads)))


@dataclass
class Summary:
    n_rows: int
    kld_sum: float
    kld_mean: float
    kld_max: float
    kld_max_row: int
    n_match: int
    same_top1: float


def summary(kl: np.ndarray, match: np.ndarray) -> Summary:
    """Mean (exactly rounded sum via math.fsum), max with lowest row, match count.

    Means and percentages are taken over every row passed in, unweighted, as
    the pages report them ("Raw benchmark data" table of the Qwen3.6 27B
    benchmark; "Quality" section of the GSQ-RCO model card).
    """
    kl = np.asarray(kl, dtype=np.float64)
    match = np.asarray(match)
    n = int(kl.shape[0])
    if n == 0:
        raise ValueError("summary over zero rows")
    s = math.fsum(kl.tolist())
    mx = -math.inf
    at = -1
    for r, v in enumerate(kl.tolist()):
        if v > mx:
            mx, at = v, r
    nm = int(np.count_nonzero(match))
    return Summary(n, s, s / n, mx, at, nm, nm / n)


from .twin import rows_scipy  # noqa: E402
from .bruteforce import bruteforce  # noqa: E402

__all__ = ["rows", "rows_scipy", "bruteforce", "summary", "Summary", "RowResults",
           "F32", "BF16", "F64", "to_f64", "bf16_bits_to_f64", "max_threads", "open_library"]
