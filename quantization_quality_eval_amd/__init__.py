"""MI355X (gfx950) quantized-vs-base logit comparison: per-token KL divergence
and same-top-1, reduced to mean / max KLD and the top-1 agreement fraction;
with next-token ids also each model's log-probability of the actual token,
reduced to perplexities, their ratio and the mean / RMS probability change;
summaries over the whole evaluation or per segment; the gradient of the KL
divergence with respect to the quantized logits; and base rows stored as
their top-K tokens plus the rest of the mass, compared with full quant rows.

This module is a thin ctypes binding over the C ABI in ``include/kld_eval.h``
(``libkldeval.so``, built from ``csrc/``). It only marshals arguments: every
step of the computation runs in the HIP kernels. PyTorch supplies device
memory (``tensor.data_ptr()``) and streams (``torch.cuda.current_stream()``).

There is no CPU fallback: if the library or a gfx950 device is missing, the
calls raise.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

from .build import build_library, library_path

KLD_DTYPE_F32 = 0
KLD_DTYPE_BF16 = 1
# conditioning flags of a row (kld_eval_copy_row_flags)
KLD_ROW_FLAG_AMPLIFIED = 1
KLD_ROW_FLAG_QUANT_MASS = 2
KLD_ROW_FLAG_CARRIED = 4

KLD_OK = 0
KLD_ERR_INVALID_ARG = -1
KLD_ERR_NO_DEVICE = -2
KLD_ERR_UNSUPPORTED_ARCH = -3
KLD_ERR_OUT_OF_MEMORY = -4
KLD_ERR_RANGE = -5
KLD_ERR_HIP = -6
KLD_ERR_BAD_HANDLE = -7
KLD_ERR_EMPTY = -8

STATUS_NAMES = {
    KLD_OK: "KLD_OK", KLD_ERR_INVALID_ARG: "KLD_ERR_INVALID_ARG", KLD_ERR_NO_DEVICE: "KLD_ERR_NO_DEVICE",
    KLD_ERR_UNSUPPORTED_ARCH: "KLD_ERR_UNSUPPORTED_ARCH", KLD_ERR_OUT_OF_MEMORY: "KLD_ERR_OUT_OF_MEMORY",
    KLD_ERR_RANGE: "KLD_ERR_RANGE", KLD_ERR_HIP: "KLD_ERR_HIP", KLD_ERR_BAD_HANDLE: "KLD_ERR_BAD_HANDLE",
    KLD_ERR_EMPTY: "KLD_ERR_EMPTY",
}


class kld_eval_summary(ctypes.Structure):
    _fields_ = [("n_rows", ctypes.c_int64), ("kld_sum", ctypes.c_double), ("kld_mean", ctypes.c_double),
                ("kld_max", ctypes.c_double), ("kld_max_row", ctypes.c_int64), ("n_match", ctypes.c_int64),
                ("same_top1", ctypes.c_double)]


class kld_eval_token_summary(ctypes.Structure):
    _fields_ = [("n_scored", ctypes.c_int64), ("n_invalid", ctypes.c_int64), ("logp_base_sum", ctypes.c_double),
                ("logp_quant_sum", ctypes.c_double), ("ppl_base", ctypes.c_double), ("ppl_quant", ctypes.c_double),
                ("ppl_ratio", ctypes.c_double), ("dp_mean", ctypes.c_double), ("dp_rms", ctypes.c_double)]


class KldEvalError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


_lib = None


def load_library(build_if_missing: bool = True):
    """Load libkldeval.so (building it from source first if it is absent)."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        if not build_if_missing:
            raise FileNotFoundError(path)
        build_library()
    lib = ctypes.CDLL(path)
    i64, i32, vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
    lib.kld_eval_create.argtypes = [ctypes.POINTER(vp), i64, i64, i32, i32]
    lib.kld_eval_rows.argtypes = [vp, vp, vp, i64, i64, vp, vp, vp, vp, vp]
    lib.kld_eval_rows_tokens.argtypes = [vp, vp, vp, vp, i64, i64, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.kld_eval_rows_timed.argtypes = [vp, vp, vp, i64, i64, vp, vp, vp, vp, vp, vp, vp]
    lib.kld_eval_reduce.argtypes = [vp, i64, ctypes.POINTER(kld_eval_summary), vp]
    lib.kld_eval_reduce_async.argtypes = [vp, i64, vp, vp]
    lib.kld_eval_reduce_tokens.argtypes = [vp, i64, ctypes.POINTER(kld_eval_token_summary), vp]
    lib.kld_eval_reduce_segments.argtypes = [vp, ctypes.POINTER(i64), i64, ctypes.POINTER(kld_eval_summary),
                                             ctypes.POINTER(kld_eval_token_summary), vp]
    lib.kld_eval_copy_lse.argtypes = [vp, i64, i64, vp, vp, vp]
    lib.kld_eval_copy_row_flags.argtypes = [vp, i64, i64, vp, vp]
    lib.kld_eval_grad.argtypes = [vp, vp, vp, i64, i64, ctypes.c_double, vp, i32, vp]
    lib.kld_eval_topk_compress.argtypes = [vp, vp, i64, i32, vp, vp, vp, vp]
    lib.kld_eval_rows_topk.argtypes = [vp, vp, vp, vp, i32, vp, i64, i64, vp, vp, vp, vp, vp]
    lib.kld_eval_grad_topk.argtypes = [vp, vp, vp, i32, vp, i64, i64, ctypes.c_double, vp, i32, vp]
    lib.kld_eval_read_probe.argtypes = [vp, vp, i64, i64, i32, vp, vp, vp, vp]
    lib.kld_eval_compare_noalloc.argtypes = [vp, vp, i64, i64, i32, i32, vp, vp, vp, vp, vp, vp]
    lib.kld_eval_destroy.argtypes = [vp]
    for f in (lib.kld_eval_create, lib.kld_eval_rows, lib.kld_eval_rows_tokens, lib.kld_eval_reduce,
              lib.kld_eval_reduce_async,
              lib.kld_eval_reduce_tokens, lib.kld_eval_reduce_segments, lib.kld_eval_copy_lse,
              lib.kld_eval_copy_row_flags,
              lib.kld_eval_grad, lib.kld_eval_topk_compress, lib.kld_eval_rows_topk, lib.kld_eval_grad_topk,
              lib.kld_eval_read_probe, lib.kld_eval_compare_noalloc, lib.kld_eval_destroy):
        f.restype = ctypes.c_int
    lib.kld_eval_last_error.argtypes = []
    lib.kld_eval_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(status: int) -> int:
    if status != KLD_OK:
        msg = load_library().kld_eval_last_error().decode(errors="replace")
        raise KldEvalError(status, msg)
    return status


# ---- same-name functions over raw pointers (integers) and a void* stream ----

def kld_eval_create(vocab: int, max_rows: int, base_dtype: int, quant_dtype: int) -> int:
    h = ctypes.c_void_p()
    _check(load_library().kld_eval_create(ctypes.byref(h), vocab, max_rows, base_dtype, quant_dtype))
    return h.value


def kld_eval_rows(h: int, base: int, quant: int, n_rows: int, row_offset: int, kld_out: int = 0,
                  match_out: int = 0, argmax_base_out: int = 0, argmax_quant_out: int = 0, stream: int = 0) -> int:
    return _check(load_library().kld_eval_rows(h, base, quant, n_rows, row_offset, kld_out or None,
                                               match_out or None, argmax_base_out or None,
                                               argmax_quant_out or None, stream or None))


def kld_eval_rows_timed(h: int, base: int, quant: int, n_rows: int, row_offset: int, kld_out: int = 0,
                        match_out: int = 0, argmax_base_out: int = 0, argmax_quant_out: int = 0, stream: int = 0,
                        start_event: int = 0, stop_event: int = 0) -> int:
    return _check(load_library().kld_eval_rows_timed(h, base, quant, n_rows, row_offset, kld_out or None,
                                                     match_out or None, argmax_base_out or None,
                                                     argmax_quant_out or None, stream or None, start_event or None,
                                                     stop_event or None))


def kld_eval_rows_tokens(h: int, base: int, quant: int, tokens: int, n_rows: int, row_offset: int,
                         kld_out: int = 0, match_out: int = 0, argmax_base_out: int = 0, argmax_quant_out: int = 0,
                         logp_base_out: int = 0, logp_quant_out: int = 0, dp_out: int = 0, stream: int = 0) -> int:
    return _check(load_library().kld_eval_rows_tokens(
        h, base, quant, tokens or None, n_rows, row_offset, kld_out or None, match_out or None,
        argmax_base_out or None, argmax_quant_out or None, logp_base_out or None, logp_quant_out or None,
        dp_out or None, stream or None))


def kld_eval_reduce_tokens(h: int, n_rows: int, stream: int = 0) -> kld_eval_token_summary:
    s = kld_eval_token_summary()
    _check(load_library().kld_eval_reduce_tokens(h, n_rows, ctypes.byref(s), stream or None))
    return s


def kld_eval_reduce_segments(h: int, offsets, stream: int = 0, want_kld: bool = True, want_tokens: bool = True):
    """Per-segment summaries for segments [offsets[s], offsets[s+1]); returns two
    ctypes arrays (or None for the one not asked for)."""
    offs = [int(o) for o in offsets]
    n = len(offs) - 1
    if n < 1:
        raise ValueError("offsets needs at least two entries")
    arr = (ctypes.c_int64 * (n + 1))(*offs)
    ks = (kld_eval_summary * n)() if want_kld else None
    ts = (kld_eval_token_summary * n)() if want_tokens else None
    _check(load_library().kld_eval_reduce_segments(h, arr, n, ks, ts, stream or None))
    return ks, ts


def kld_eval_reduce(h: int, n_rows: int, stream: int = 0) -> kld_eval_summary:
    s = kld_eval_summary()
    _check(load_library().kld_eval_reduce(h, n_rows, ctypes.byref(s), stream or None))
    return s


def kld_eval_reduce_async(h: int, n_rows: int, out: int, stream: int = 0) -> int:
    """out: address of device memory or pinned host memory for one kld_eval_summary."""
    return _check(load_library().kld_eval_reduce_async(h, n_rows, out or None, stream or None))


def summary_from_bytes(buf) -> Summary:
    """Summary from the bytes of a kld_eval_summary (a uint8 tensor, or bytes)."""
    size = ctypes.sizeof(kld_eval_summary)
    raw = bytes(buf[:size].cpu().tolist()) if hasattr(buf, "cpu") else bytes(buf)[:size]
    return _summary(kld_eval_summary.from_buffer_copy(raw))


def kld_eval_copy_lse(h: int, row_offset: int, n_rows: int, lse_base_out: int = 0, lse_quant_out: int = 0,
                      stream: int = 0) -> int:
    return _check(load_library().kld_eval_copy_lse(h, row_offset, n_rows, lse_base_out or None,
                                                   lse_quant_out or None, stream or None))


def kld_eval_copy_row_flags(h: int, row_offset: int, n_rows: int, flags_out: int, stream: int = 0) -> int:
    return _check(load_library().kld_eval_copy_row_flags(h, row_offset, n_rows, flags_out or None, stream or None))


def kld_eval_grad(h: int, base: int, quant: int, n_rows: int, row_offset: int, scale: float, grad_out: int,
                  grad_dtype: int, stream: int = 0) -> int:
    return _check(load_library().kld_eval_grad(h, base, quant, n_rows, row_offset, float(scale), grad_out or None,
                                               grad_dtype, stream or None))


def kld_eval_topk_compress(h: int, base: int, n_rows: int, k: int, idx_out: int, logp_out: int, rest_out: int,
                           stream: int = 0) -> int:
    return _check(load_library().kld_eval_topk_compress(h, base, n_rows, k, idx_out or None, logp_out or None,
                                                        rest_out or None, stream or None))


def kld_eval_rows_topk(h: int, topk_idx: int, topk_logp: int, topk_rest: int, k: int, quant: int, n_rows: int,
                       row_offset: int, kld_out: int = 0, match_out: int = 0, argmax_base_out: int = 0,
                       argmax_quant_out: int = 0, stream: int = 0) -> int:
    return _check(load_library().kld_eval_rows_topk(h, topk_idx or None, topk_logp or None, topk_rest or None, k,
                                                    quant or None, n_rows, row_offset, kld_out or None,
                                                    match_out or None, argmax_base_out or None,
                                                    argmax_quant_out or None, stream or None))


def kld_eval_grad_topk(h: int, topk_idx: int, topk_logp: int, k: int, quant: int, n_rows: int, row_offset: int,
                       scale: float, grad_out: int, grad_dtype: int, stream: int = 0) -> int:
    return _check(load_library().kld_eval_grad_topk(h, topk_idx or None, topk_logp or None, k, quant or None, n_rows,
                                                    row_offset, float(scale), grad_out or None, grad_dtype,
                                                    stream or None))


def kld_eval_read_probe(a: int, b: int, n_rows: int, row_bytes: int, waves_per_row: int, sink: int,
                        stream: int = 0, start_event: int = 0, stop_event: int = 0) -> int:
    return _check(load_library().kld_eval_read_probe(a or None, b or None, n_rows, row_bytes, waves_per_row,
                                                     sink or None, stream or None, start_event or None,
                                                     stop_event or None))


def read_probe(a, b=None, stream=None, waves_per_row: int = 4, start_event=None, stop_event=None):
    """Read-bandwidth probe over the rows of device tensors a (and b, same
    shape), with 1 or 4 waves per row: returns the per-row XOR of their 32-bit
    words (uint32 tensor, as int32), written asynchronously on ``stream``.
    ``start_event`` / ``stop_event`` (torch.cuda.Event, already recorded once)
    are recorded by the probe's launch itself."""
    import torch
    if a.dim() != 2 or not a.is_cuda or not a.is_contiguous():
        raise ValueError("a: expected a contiguous 2-D device tensor")
    if b is not None and (b.shape != a.shape or b.dtype != a.dtype or b.device != a.device or not b.is_contiguous()):
        raise ValueError("b: expected a contiguous tensor like a")
    n = a.shape[0]
    sink = torch.empty(n, dtype=torch.int32, device=a.device)
    kld_eval_read_probe(a.data_ptr(), 0 if b is None else b.data_ptr(), n, a.shape[1] * a.element_size(),
                        waves_per_row, sink.data_ptr(), _stream_ptr(stream, a.device),
                        _event_ptr(start_event, "start_event", a.device), _event_ptr(stop_event, "stop_event", a.device))
    return sink


def kld_eval_compare_noalloc(base: int, quant: int, vocab: int, n_rows: int, base_dtype: int, quant_dtype: int,
                             kld_out: int, match_out: int, argmax_base_out: int = 0, argmax_quant_out: int = 0,
                             summary_out: int = 0, stream: int = 0) -> int:
    return _check(load_library().kld_eval_compare_noalloc(base, quant, vocab, n_rows, base_dtype, quant_dtype,
                                                          kld_out or None, match_out or None, argmax_base_out or None,
                                                          argmax_quant_out or None, summary_out or None,
                                                          stream or None))


def kld_eval_destroy(h: int) -> int:
    return _check(load_library().kld_eval_destroy(h))


def kld_eval_last_error() -> str:
    return load_library().kld_eval_last_error().decode(errors="replace")


# ---- torch-facing convenience wrapper ----

@dataclass
class Summary:
    n_rows: int
    kld_sum: float
    kld_mean: float
    kld_max: float
    kld_max_row: int
    n_match: int
    same_top1: float


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


def _summary(s: kld_eval_summary) -> Summary:
    return Summary(s.n_rows, s.kld_sum, s.kld_mean, s.kld_max, s.kld_max_row, s.n_match, s.same_top1)


def _token_summary(s: kld_eval_token_summary) -> TokenSummary:
    return TokenSummary(s.n_scored, s.n_invalid, s.logp_base_sum, s.logp_quant_sum, s.ppl_base, s.ppl_quant,
                        s.ppl_ratio, s.dp_mean, s.dp_rms)


def _dtype_code(dt) -> int:
    import torch
    if dt in (torch.float32, "f32", KLD_DTYPE_F32):
        return KLD_DTYPE_F32
    if dt in (torch.bfloat16, "bf16", KLD_DTYPE_BF16):
        return KLD_DTYPE_BF16
    raise ValueError(f"unsupported dtype {dt}")


def _event_ptr(event, name, device=None) -> int:
    """The hipEvent_t of a torch.cuda.Event (0 for None). torch creates the
    underlying event at its first record, so an event that was never recorded
    has none yet and is refused; so is one made on another device than
    ``device`` (the launch that records it runs there)."""
    if event is None:
        return 0
    ptr = int(event.cuda_event)
    if not ptr:
        raise ValueError(f"{name}: the event has no HIP event yet (record it once first)")
    if device is not None and event.device is not None and event.device != device:
        raise ValueError(f"{name}: expected an event on {device}, got {event.device}")
    return ptr


def _stream_ptr(stream, device) -> int:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return int(stream.cuda_stream)


class Evaluator:
    """One handle: vocab size, row capacity and the two input dtypes are fixed."""

    def __init__(self, vocab: int, max_rows: int, base_dtype="bf16", quant_dtype="bf16", device=None):
        import torch
        self.device = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
        self.vocab = int(vocab)
        self.max_rows = int(max_rows)
        self.base_code = _dtype_code(base_dtype)
        self.quant_code = _dtype_code(quant_dtype)
        with torch.cuda.device(self.device):
            self.handle = kld_eval_create(self.vocab, self.max_rows, self.base_code, self.quant_code)

    def _check_input(self, t, code, name):
        import torch
        want = torch.float32 if code == KLD_DTYPE_F32 else torch.bfloat16
        if t.dtype != want:
            raise TypeError(f"{name}: expected {want}, got {t.dtype}")
        if t.device != self.device:
            raise ValueError(f"{name}: expected a tensor on {self.device}, got {t.device}")
        if t.dim() != 2 or t.shape[1] != self.vocab or not t.is_contiguous():
            raise ValueError(f"{name}: expected a contiguous [n, {self.vocab}] tensor, got {tuple(t.shape)}")

    def _ptr(self, t, n, dtype, name):
        """Device address of an optional per-row array (0 for None). Every such
        array is read or written by the kernels, so it must live on this
        handle's device: a host tensor's address would reach a kernel."""
        if t is None:
            return 0
        if t.dtype != dtype or t.numel() < n or not t.is_contiguous():
            raise ValueError(f"{name}: expected a contiguous {dtype} tensor with >= {n} elements")
        if t.device != self.device:
            raise ValueError(f"{name}: expected a tensor on {self.device}, got {t.device}")
        return t.data_ptr()

    def rows(self, base, quant, row_offset: int = 0, kld_out=None, match_out=None, argmax_base_out=None,
             argmax_quant_out=None, stream=None, tokens=None, logp_base_out=None, logp_quant_out=None,
             dp_out=None, start_event=None, stop_event=None) -> None:
        """Evaluate row pairs into handle rows [row_offset, row_offset + n). With
        ``tokens`` (int32 [n] on the device: the id of the token that follows
        each position, -1 for none) the token-conditioned values are computed in
        the same pass. ``start_event`` / ``stop_event`` (torch.cuda.Event with
        timing, already created by a first record) are recorded by the row
        kernel's launch itself (kld_eval_rows_timed); not with ``tokens``."""
        import torch
        self._check_input(base, self.base_code, "base")
        self._check_input(quant, self.quant_code, "quant")
        if base.shape != quant.shape:
            raise ValueError("base and quant shapes differ")
        n = base.shape[0]
        if start_event is not None or stop_event is not None:
            if tokens is not None or logp_base_out is not None or logp_quant_out is not None or dp_out is not None:
                raise ValueError("start_event / stop_event: not with next-token ids")
            kld_eval_rows_timed(self.handle, base.data_ptr(), quant.data_ptr(), n, row_offset,
                                self._ptr(kld_out, n, torch.float32, "kld_out"),
                                self._ptr(match_out, n, torch.uint8, "match_out"),
                                self._ptr(argmax_base_out, n, torch.int32, "argmax_base_out"),
                                self._ptr(argmax_quant_out, n, torch.int32, "argmax_quant_out"),
                                _stream_ptr(stream, self.device), _event_ptr(start_event, "start_event", self.device),
                                _event_ptr(stop_event, "stop_event", self.device))
            return
        if tokens is not None:
            if tokens.device != self.device or tokens.dim() != 1 or tokens.shape[0] != n:
                raise ValueError(f"tokens: expected a 1-d tensor of {n} ids on {self.device}")
        kld_eval_rows_tokens(self.handle, base.data_ptr(), quant.data_ptr(),
                             self._ptr(tokens, n, torch.int32, "tokens"), n, row_offset,
                             self._ptr(kld_out, n, torch.float32, "kld_out"),
                             self._ptr(match_out, n, torch.uint8, "match_out"),
                             self._ptr(argmax_base_out, n, torch.int32, "argmax_base_out"),
                             self._ptr(argmax_quant_out, n, torch.int32, "argmax_quant_out"),
                             self._ptr(logp_base_out, n, torch.float32, "logp_base_out"),
                             self._ptr(logp_quant_out, n, torch.float32, "logp_quant_out"),
                             self._ptr(dp_out, n, torch.float32, "dp_out"),
                             _stream_ptr(stream, self.device))

    def reduce(self, n_rows: int, stream=None) -> Summary:
        return _summary(kld_eval_reduce(self.handle, n_rows, _stream_ptr(stream, self.device)))

    def reduce_async(self, n_rows: int, out=None, stream=None):
        """Enqueue the reduction of rows [0, n_rows) and return at once; the
        summary's bytes land in ``out`` (a uint8 tensor of at least
        sizeof(kld_eval_summary) bytes, pinned host memory by default, or on
        this handle's device) when the stream reaches it: decode them with
        ``summary_from_bytes`` after synchronizing."""
        import torch
        size = ctypes.sizeof(kld_eval_summary)
        if out is None:
            out = torch.empty(size, dtype=torch.uint8, pin_memory=True)
        if out.dtype != torch.uint8 or out.numel() < size or not out.is_contiguous():
            raise ValueError(f"out: expected a contiguous uint8 tensor of >= {size} bytes")
        if out.device.type == "cpu":
            if not out.is_pinned():
                raise ValueError("out: a host tensor must be pinned (the device writes it)")
        elif out.device != self.device:
            raise ValueError(f"out: expected a tensor on {self.device} or pinned host memory, got {out.device}")
        kld_eval_reduce_async(self.handle, n_rows, out.data_ptr(), _stream_ptr(stream, self.device))
        return out

    def reduce_tokens(self, n_rows: int, stream=None, allow_invalid: bool = False) -> TokenSummary:
        """Token-conditioned summary of rows [0, n_rows). Raises ValueError when
        some token id was >= vocab, unless ``allow_invalid``."""
        t = _token_summary(kld_eval_reduce_tokens(self.handle, n_rows, _stream_ptr(stream, self.device)))
        if t.n_invalid and not allow_invalid:
            raise ValueError(f"{t.n_invalid} token ids were >= vocab ({self.vocab}); those rows were not scored")
        return t

    def reduce_segments(self, offsets, stream=None):
        """Per-segment (Summary, TokenSummary) pairs for rows [offsets[s], offsets[s+1])."""
        ks, ts = kld_eval_reduce_segments(self.handle, offsets, _stream_ptr(stream, self.device))
        return [(_summary(k), _token_summary(t)) for k, t in zip(ks, ts)]

    def copy_lse(self, row_offset: int, n_rows: int, lse_base_out=None, lse_quant_out=None, stream=None) -> None:
        import torch
        kld_eval_copy_lse(self.handle, row_offset, n_rows,
                          self._ptr(lse_base_out, n_rows, torch.float32, "lse_base_out"),
                          self._ptr(lse_quant_out, n_rows, torch.float32, "lse_quant_out"),
                          _stream_ptr(stream, self.device))

    def row_flags(self, row_offset: int, n_rows: int, out=None, stream=None):
        """Conditioning flags of handle rows [row_offset, row_offset + n) as a
        uint8 tensor (KLD_ROW_FLAG_* bits; nonzero: the row was evaluated a
        second time in float64)."""
        import torch
        if out is None:
            out = torch.empty(max(n_rows, 0), dtype=torch.uint8, device=self.device)
        kld_eval_copy_row_flags(self.handle, row_offset, n_rows, self._ptr(out, n_rows, torch.uint8, "out"),
                                _stream_ptr(stream, self.device))
        return out

    def grad(self, base, quant, row_offset: int = 0, scale: float = 1.0, out=None, dtype="f32", stream=None):
        """d KL / d z_quant = scale * (q - p) for rows that ``rows`` already
        evaluated into [row_offset, row_offset + n); returns ``out`` (allocated
        as [n, vocab] of ``dtype`` if None)."""
        import torch
        self._check_input(base, self.base_code, "base")
        self._check_input(quant, self.quant_code, "quant")
        if base.shape != quant.shape:
            raise ValueError("base and quant shapes differ")
        code = _dtype_code(dtype)
        want = torch.float32 if code == KLD_DTYPE_F32 else torch.bfloat16
        n = base.shape[0]
        if out is None:
            out = torch.empty((n, self.vocab), dtype=want, device=self.device)
        if out.dtype != want or out.device != self.device or not out.is_contiguous() or out.numel() < n * self.vocab:
            raise ValueError(f"out: expected a contiguous {want} tensor with >= {n * self.vocab} elements on "
                             f"{self.device}")
        kld_eval_grad(self.handle, base.data_ptr(), quant.data_ptr(), n, row_offset, scale, out.data_ptr(), code,
                      _stream_ptr(stream, self.device))
        return out

    def topk_compress(self, base, k: int, stream=None):
        """Stored top-k + rest form of base rows: (idx int32 [n, k], logp float32
        [n, k], rest float32 [n]) tensors on the device."""
        import torch
        self._check_input(base, self.base_code, "base")
        n = base.shape[0]
        idx = torch.empty((n, k), dtype=torch.int32, device=self.device)
        logp = torch.empty((n, k), dtype=torch.float32, device=self.device)
        rest = torch.empty(n, dtype=torch.float32, device=self.device)
        kld_eval_topk_compress(self.handle, base.data_ptr(), n, k, idx.data_ptr(), logp.data_ptr(), rest.data_ptr(),
                               _stream_ptr(stream, self.device))
        return idx, logp, rest

    def rows_topk(self, idx, logp, rest, quant, row_offset: int = 0, kld_out=None, match_out=None,
                  argmax_base_out=None, argmax_quant_out=None, stream=None) -> None:
        """Coarsened KL of full quant rows from stored top-k base rows, into handle
        rows [row_offset, row_offset + n) like ``rows``."""
        import torch
        self._check_input(quant, self.quant_code, "quant")
        n = quant.shape[0]
        self._check_topk(idx, logp, rest, n)
        kld_eval_rows_topk(self.handle, idx.data_ptr(), logp.data_ptr(), rest.data_ptr(), idx.shape[1],
                           quant.data_ptr(), n, row_offset,
                           self._ptr(kld_out, n, torch.float32, "kld_out"),
                           self._ptr(match_out, n, torch.uint8, "match_out"),
                           self._ptr(argmax_base_out, n, torch.int32, "argmax_base_out"),
                           self._ptr(argmax_quant_out, n, torch.int32, "argmax_quant_out"),
                           _stream_ptr(stream, self.device))

    def grad_topk(self, idx, logp, quant, row_offset: int = 0, scale: float = 1.0, out=None, dtype="f32",
                  stream=None):
        """d KL_k / d z_quant for rows that ``rows_topk`` already evaluated into
        [row_offset, row_offset + n) from the same stored rows (their rest mass
        enters through the factors that call saved); returns ``out``
        (allocated as [n, vocab] of ``dtype`` if None)."""
        import torch
        self._check_input(quant, self.quant_code, "quant")
        n = quant.shape[0]
        self._check_topk(idx, logp, None, n)
        code = _dtype_code(dtype)
        want = torch.float32 if code == KLD_DTYPE_F32 else torch.bfloat16
        if out is None:
            out = torch.empty((n, self.vocab), dtype=want, device=self.device)
        if out.dtype != want or out.device != self.device or not out.is_contiguous() or out.numel() < n * self.vocab:
            raise ValueError(f"out: expected a contiguous {want} tensor with >= {n * self.vocab} elements on "
                             f"{self.device}")
        kld_eval_grad_topk(self.handle, idx.data_ptr(), logp.data_ptr(), idx.shape[1], quant.data_ptr(), n,
                           row_offset, scale, out.data_ptr(), code, _stream_ptr(stream, self.device))
        return out

    def _check_topk(self, idx, logp, rest, n):
        import torch
        if idx.dim() != 2 or idx.shape[0] != n or logp.shape != idx.shape or (rest is not None and rest.shape != (n,)):
            raise ValueError("idx/logp must be [n, k] and rest [n] for the n quant rows")
        for name, t, dt in (("idx", idx, torch.int32), ("logp", logp, torch.float32), ("rest", rest, torch.float32)):
            if t is None:
                continue
            if t.dtype != dt or t.device != self.device or not t.is_contiguous():
                raise ValueError(f"{name}: expected a contiguous {dt} tensor on {self.device}")

    def close(self) -> None:
        if getattr(self, "handle", None):
            h, self.handle = self.handle, None
            kld_eval_destroy(h)

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def compare(base, quant, stream=None):
    """One-shot helper: per-token (kld, match, argmax_base, argmax_quant) tensors and the summary."""
    import torch
    n, v = base.shape
    dev = base.device
    kld = torch.empty(n, dtype=torch.float32, device=dev)
    match = torch.empty(n, dtype=torch.uint8, device=dev)
    ab = torch.empty(n, dtype=torch.int32, device=dev)
    aq = torch.empty(n, dtype=torch.int32, device=dev)
    with Evaluator(v, max(n, 1), base.dtype, quant.dtype, device=dev) as ev:
        ev.rows(base, quant, 0, kld, match, ab, aq, stream=stream)
        summ = ev.reduce(n, stream=stream) if n > 0 else None
    return kld, match, ab, aq, summ


def compare_tokens(base, quant, tokens, stream=None, allow_invalid: bool = False):
    """One-shot helper with next-token ids: per-token (kld, match, logp_base,
    logp_quant, dp) tensors, the summary and the token summary."""
    import torch
    n, v = base.shape
    dev = base.device
    f = dict(dtype=torch.float32, device=dev)
    kld, lpb, lpq, dp = (torch.empty(n, **f) for _ in range(4))
    match = torch.empty(n, dtype=torch.uint8, device=dev)
    with Evaluator(v, max(n, 1), base.dtype, quant.dtype, device=dev) as ev:
        ev.rows(base, quant, 0, kld, match, stream=stream, tokens=tokens, logp_base_out=lpb, logp_quant_out=lpq,
                dp_out=dp)
        summ = ev.reduce(n, stream=stream) if n > 0 else None
        tsum = ev.reduce_tokens(n, stream=stream, allow_invalid=allow_invalid) if n > 0 else None
    return kld, match, lpb, lpq, dp, summ, tsum


__all__ = ["Evaluator", "Summary", "TokenSummary", "compare", "compare_tokens", "KldEvalError", "kld_eval_create",
           "kld_eval_rows", "kld_eval_rows_tokens", "kld_eval_reduce", "kld_eval_reduce_tokens",
           "kld_eval_reduce_segments", "kld_eval_copy_lse", "kld_eval_copy_row_flags", "kld_eval_grad", "kld_eval_topk_compress",
           "kld_eval_rows_topk", "kld_eval_grad_topk", "kld_eval_read_probe", "read_probe", "kld_eval_destroy",
           "kld_eval_compare_noalloc", "kld_eval_reduce_async", "summary_from_bytes",
           "kld_eval_last_error",
           "load_library", "build_library", "library_path", "KLD_DTYPE_F32", "KLD_DTYPE_BF16",
           "KLD_ROW_FLAG_AMPLIFIED", "KLD_ROW_FLAG_QUANT_MASS", "KLD_ROW_FLAG_CARRIED"]
