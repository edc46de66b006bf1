"""The C ABI without a GPU: the library loads, exports every declared symbol,
and rejects bad arguments before touching any device."""
import ctypes
import os
import re

import numpy as np
import pytest

import quantization_quality_eval_amd as qqe

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "kld_eval.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kld_eval_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for want in ["kld_eval_create", "kld_eval_rows", "kld_eval_reduce", "kld_eval_destroy",
                 "kld_eval_last_error", "kld_eval_copy_lse", "kld_eval_rows_tokens", "kld_eval_reduce_tokens",
                 "kld_eval_reduce_segments", "kld_eval_grad", "kld_eval_topk_compress", "kld_eval_rows_topk",
                 "kld_eval_grad_topk", "kld_eval_read_probe", "kld_eval_copy_row_flags", "kld_eval_rows_timed"]:
        assert want in names


def test_library_exports_every_declared_symbol():
    lib = qqe.load_library()
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_exported_symbols_match_nm():
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", qqe.library_path()], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT (kld_eval_\w+)", out))
    assert exported == set(declared_functions())


def _raw():
    return qqe.load_library()


def test_create_rejects_bad_arguments_before_device():
    lib = _raw()
    h = ctypes.c_void_p(1234)
    assert lib.kld_eval_create(None, 10, 10, 0, 0) == qqe.KLD_ERR_INVALID_ARG
    for vocab, rows, bt, qt in [(0, 10, 0, 0), (-5, 10, 0, 0), (2**31, 10, 0, 0), (10, 0, 0, 0),
                                (10, -1, 0, 0), (10, 10, 2, 0), (10, 10, 0, -1), (10, 2**41, 1, 1)]:
        assert lib.kld_eval_create(ctypes.byref(h), vocab, rows, bt, qt) == qqe.KLD_ERR_INVALID_ARG
        assert h.value is None            # *out cleared on failure
        assert qqe.kld_eval_last_error()


def _no_gpu():
    try:
        import torch
        return not torch.cuda.is_available()
    except Exception:
        return True


@pytest.mark.skipif(not _no_gpu(), reason="checks the no-device path")
def test_create_without_device_reports_no_device():
    h = ctypes.c_void_p()
    st = _raw().kld_eval_create(ctypes.byref(h), 151936, 8192, qqe.KLD_DTYPE_BF16, qqe.KLD_DTYPE_BF16)
    assert st == qqe.KLD_ERR_NO_DEVICE
    assert "device" in qqe.kld_eval_last_error()
    with pytest.raises(qqe.KldEvalError) as ei:
        qqe.kld_eval_create(100, 4, 0, 0)
    assert ei.value.status == qqe.KLD_ERR_NO_DEVICE


def test_calls_on_null_or_foreign_handles():
    lib = _raw()
    s = qqe.kld_eval_summary()
    assert lib.kld_eval_rows(None, 1, 1, 4, 0, None, None, None, None, None) == qqe.KLD_ERR_BAD_HANDLE
    assert lib.kld_eval_reduce(None, 4, ctypes.byref(s), None) == qqe.KLD_ERR_BAD_HANDLE
    assert lib.kld_eval_copy_lse(None, 0, 4, None, None, None) == qqe.KLD_ERR_BAD_HANDLE
    assert lib.kld_eval_copy_row_flags(None, 0, 4, None, None) == qqe.KLD_ERR_BAD_HANDLE
    ts = qqe.kld_eval_token_summary()
    assert lib.kld_eval_rows_tokens(None, 1, 1, 1, 4, 0, None, None, None, None, None, None, None,
                                    None) == qqe.KLD_ERR_BAD_HANDLE
    assert lib.kld_eval_rows_timed(None, 1, 1, 4, 0, None, None, None, None, None, None,
                                   None) == qqe.KLD_ERR_BAD_HANDLE
    assert lib.kld_eval_reduce_tokens(None, 4, ctypes.byref(ts), None) == qqe.KLD_ERR_BAD_HANDLE
    offs = (ctypes.c_int64 * 2)(0, 4)
    assert lib.kld_eval_reduce_segments(None, offs, 1, None, None, None) == qqe.KLD_ERR_BAD_HANDLE
    assert lib.kld_eval_grad(None, 1, 1, 4, 0, 1.0, 1, 0, None) == qqe.KLD_ERR_BAD_HANDLE
    assert lib.kld_eval_topk_compress(None, 1, 4, 8, 1, 1, 1, None) == qqe.KLD_ERR_BAD_HANDLE
    assert lib.kld_eval_rows_topk(None, 1, 1, 1, 8, 1, 4, 0, None, None, None, None, None) == qqe.KLD_ERR_BAD_HANDLE
    assert lib.kld_eval_grad_topk(None, 1, 1, 8, 1, 4, 0, 1.0, 1, 0, None) == qqe.KLD_ERR_BAD_HANDLE
    assert lib.kld_eval_destroy(None) == qqe.KLD_OK
    # a pointer that was never returned by kld_eval_create is recognised without being dereferenced
    fake = ctypes.create_string_buffer(256)
    addr = ctypes.addressof(fake)
    assert lib.kld_eval_rows(addr, 1, 1, 4, 0, None, None, None, None, None) == qqe.KLD_ERR_BAD_HANDLE
    assert lib.kld_eval_destroy(addr) == qqe.KLD_ERR_BAD_HANDLE
    assert "handle" in qqe.kld_eval_last_error()


def test_read_probe_rejects_bad_arguments_before_device():
    lib = _raw()
    assert lib.kld_eval_read_probe(None, None, 0, 16, 4, None, None, None, None) == qqe.KLD_OK
    assert lib.kld_eval_read_probe(16, None, -1, 16, 4, 16, None, None, None) == qqe.KLD_ERR_INVALID_ARG
    for row_bytes in (0, -16, 24):
        assert lib.kld_eval_read_probe(16, None, 4, row_bytes, 4, 16, None, None, None) == qqe.KLD_ERR_INVALID_ARG
    for waves in (0, 2, 3, 8, -1):
        assert lib.kld_eval_read_probe(16, None, 4, 16, waves, 16, None, None, None) == qqe.KLD_ERR_INVALID_ARG
    assert lib.kld_eval_read_probe(None, None, 4, 16, 1, 16, None, None, None) == qqe.KLD_ERR_INVALID_ARG
    assert lib.kld_eval_read_probe(16, None, 4, 16, 1, None, None, None, None) == qqe.KLD_ERR_INVALID_ARG
    assert lib.kld_eval_read_probe(8, None, 4, 16, 4, 16, None, None, None) == qqe.KLD_ERR_INVALID_ARG   # misaligned a
    assert lib.kld_eval_read_probe(16, 24, 4, 16, 4, 16, None, None, None) == qqe.KLD_ERR_INVALID_ARG    # misaligned b
    assert "read_probe" in qqe.kld_eval_last_error()


def test_status_values_match_header():
    text = open(HEADER).read()
    for name, val in re.findall(r"(KLD_(?:OK|ERR_\w+))\s*=\s*(-?\d+)", text):
        assert getattr(qqe, name) == int(val), name
    for name, val in re.findall(r"(KLD_DTYPE_\w+)\s*=\s*(\d+)", text):
        assert getattr(qqe, name) == int(val), name
    flags = re.findall(r"(KLD_ROW_FLAG_\w+)\s*=\s*(\d+)", text)
    assert len(flags) == 3
    for name, val in flags:
        assert getattr(qqe, name) == int(val), name


def test_summary_struct_layout():
    # 7 eight-byte fields, no padding, in header order
    assert ctypes.sizeof(qqe.kld_eval_summary) == 56
    names = [f[0] for f in qqe.kld_eval_summary._fields_]
    text = open(HEADER).read()
    body = text[text.index("typedef struct kld_eval_summary"):text.index("} kld_eval_summary;")]
    assert names == re.findall(r"(?:int64_t|double)\s+(\w+);", body)


def test_token_summary_struct_layout():
    assert ctypes.sizeof(qqe.kld_eval_token_summary) == 72
    names = [f[0] for f in qqe.kld_eval_token_summary._fields_]
    text = open(HEADER).read()
    body = text[text.index("typedef struct kld_eval_token_summary"):text.index("} kld_eval_token_summary;")]
    assert names == re.findall(r"(?:int64_t|double)\s+(\w+);", body)


def test_product_path_has_no_oracle_or_cpu_fallback():
    """The binding and the HIP sources never import, call or link the oracle."""
    pkg = os.path.dirname(qqe.__file__)
    for root, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(root, f)).read()
                assert "oracle" not in text.lower(), f
                assert "import numpy" not in text, f


def test_binding_rejects_outputs_on_another_device():
    """Every per-row array handed to the library is written or read by a
    kernel: a host tensor (or one on another device) is refused before any
    call, so its address never reaches a kernel."""
    import torch
    ev = qqe.Evaluator.__new__(qqe.Evaluator)   # no handle: only the argument checks run
    ev.device = torch.device("cuda", 0)
    host = torch.empty(8, dtype=torch.float32)
    with pytest.raises(ValueError, match="expected a tensor on cuda:0"):
        ev._ptr(host, 8, torch.float32, "kld_out")
    with pytest.raises(ValueError):
        ev._ptr(torch.empty(8, dtype=torch.int32), 8, torch.float32, "kld_out")
    with pytest.raises(ValueError):
        ev._ptr(torch.empty(4, dtype=torch.float32), 8, torch.float32, "kld_out")
    assert ev._ptr(None, 8, torch.float32, "kld_out") == 0


@pytest.mark.skipif(os.environ.get("KLD_SANITIZED") != "1", reason="only in the sanitizer run (tests/run_sanitized.py)")
def test_sanitizer_run_loads_instrumented_builds():
    """Under tests/run_sanitized.py the library and the oracle in use are the
    AddressSanitizer builds (their code calls the ASan runtime's checks)."""
    import subprocess

    import oracle
    from oracle.build import oracle_library_path
    for path in (qqe.library_path(), oracle_library_path()):
        assert path.endswith("_asan.so"), path
        undefined = subprocess.run(["nm", "-D", "--undefined-only", path], capture_output=True, text=True,
                                   check=True).stdout
        assert "__asan_report" in undefined, path
    assert oracle.rows(np.zeros((1, 4), np.float32), np.zeros((1, 4), np.float32)).kl[0] == 0.0


def test_binding_refuses_uncreated_or_foreign_timing_events():
    """Timing events reach a kernel launch, so the binding refuses one that
    has no HIP event yet (never recorded) or belongs to another device, before
    any call into the library."""
    import torch

    class Event:  # the two attributes the binding reads from a torch.cuda.Event
        def __init__(self, ptr, device):
            self.cuda_event, self.device = ptr, device

    d0, d1 = torch.device("cuda:0"), torch.device("cuda:1")
    assert qqe._event_ptr(None, "start_event", d0) == 0
    assert qqe._event_ptr(Event(4096, d0), "start_event", d0) == 4096
    with pytest.raises(ValueError, match="record it once"):
        qqe._event_ptr(Event(0, d0), "start_event", d0)
    with pytest.raises(ValueError, match="expected an event on cuda:0"):
        qqe._event_ptr(Event(4096, d1), "stop_event", d0)
