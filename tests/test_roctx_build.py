"""The tracing build (every C-ABI call inside a named roctx range) on the CPU:
it compiles from the same sources, links the roctx library while the default
build does not, exports the same symbols, and its calls run with no profiler
attached."""
import os
import re
import subprocess
import sys

import pytest

import quantization_quality_eval_amd as qqe
from quantization_quality_eval_amd.build import build_traced_library
from tests.test_abi import declared_functions

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def traced(tmp_path_factory):
    return build_traced_library(str(tmp_path_factory.mktemp("roctx") / "libkldeval_roctx.so"))


def _needed(path):
    out = subprocess.run(["readelf", "-d", path], capture_output=True, text=True, check=True).stdout
    return re.findall(r"Shared library: \[([^\]]+)\]", out)


def _nm(path, *flags):
    return subprocess.run(["nm", "-D", *flags, path], capture_output=True, text=True, check=True).stdout


def test_only_the_traced_build_links_roctx(traced):
    assert any("roctx" in n for n in _needed(traced))
    assert not any("roctx" in n for n in _needed(qqe.library_path()))
    undefined = _nm(traced, "--undefined-only")
    assert "roctxRangePushA" in undefined and "roctxRangePop" in undefined
    assert "roctx" not in _nm(qqe.library_path(), "--undefined-only")


def test_traced_build_exports_the_same_boundary(traced):
    exported = set(re.findall(r"\bT (kld_eval_\w+)", _nm(traced, "--defined-only")))
    assert exported == set(declared_functions())


def test_traced_calls_run_without_a_profiler(traced):
    # a child process loads the traced library through KLD_EVAL_LIBRARY and
    # makes calls that return before any device work (argument errors)
    code = (
        "import ctypes, quantization_quality_eval_amd as qqe\n"
        "lib = qqe.load_library(build_if_missing=False)\n"
        "import os; assert qqe.library_path() == os.environ['KLD_EVAL_LIBRARY']\n"
        "h = ctypes.c_void_p()\n"
        "assert lib.kld_eval_create(ctypes.byref(h), 0, 10, 0, 0) == qqe.KLD_ERR_INVALID_ARG\n"
        "assert lib.kld_eval_destroy(None) == qqe.KLD_OK\n"
        "assert qqe.kld_eval_last_error()\n"
        "print('traced ok')\n"
    )
    env = dict(os.environ, KLD_EVAL_LIBRARY=traced)
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    assert "traced ok" in r.stdout
