"""Compile the HIP sources into the in-tree shared library libkldeval.so (gfx950)."""
from __future__ import annotations

import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
SOURCES = ["kld_eval_api.hip", "kld_row.hip", "kld_reduce.hip", "kld_grad.hip", "kld_topk.hip", "kld_probe.hip"]
ARCH = "gfx950"


def library_path() -> str:
    """The in-tree library, or the build named by KLD_EVAL_LIBRARY (for
    instance the sanitizer build the host-side tests run against)."""
    return os.environ.get("KLD_EVAL_LIBRARY") or os.path.join(PKG, "libkldeval.so")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm under /opt/rocm)")


def compile_command(out: str) -> list[str]:
    return [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            # packed fp32 VALU forms are kept out of the generated code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # no implicit fusion: the kernels state every fma they rely on, and the
            # per-token terms must use exactly the rounded values fed to the exponentials
            "-ffp-contract=off",
            "-Wall", "-Wno-unused-command-line-argument",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC,
            *[os.path.join(CSRC, s) for s in SOURCES], "-o", out]


# Host-side instrumentation only (each -fsanitize= after -Xarch_host): the GPU
# code of a sanitizer build is the same as the normal build's.
SANITIZE_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=undefined",
                 "-Xarch_host", "-g"]


def build_sanitized_library(out: str, verbose: bool = False) -> str:
    """The same library with its host code (argument validation, handle
    registry, events, workspace growth) built with AddressSanitizer and
    UndefinedBehaviorSanitizer, into ``out``. It needs clang's ASan runtime
    loaded first (LD_PRELOAD), as tests/run_sanitized.py does."""
    tmp = out + ".tmp"
    cmd = compile_command(tmp)
    cmd = cmd[:1] + SANITIZE_HOST + cmd[1:]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


# Tracing build: every call of the C ABI inside a named roctx range, for
# rocprofv3 --marker-trace (the kernels are the same as the normal build's).
ROCTX = ["-DKLD_EVAL_ROCTX", "-L/opt/rocm/lib", "-lrocprofiler-sdk-roctx", "-Wl,-rpath,/opt/rocm/lib"]


def traced_library_path() -> str:
    return os.path.join(PKG, "libkldeval_roctx.so")


def build_traced_library(out: str | None = None, verbose: bool = False) -> str:
    """The library with roctx ranges around its calls, into ``out`` (by
    default libkldeval_roctx.so beside the normal build); load it through
    KLD_EVAL_LIBRARY. The default build has no roctx dependency."""
    out = out or traced_library_path()
    tmp = out + ".tmp"
    cmd = compile_command(tmp) + ROCTX
    if verbose:
        print(" ".join(cmd), flush=True)
    os.makedirs(os.path.dirname(os.path.abspath(out)), exist_ok=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build_library(verbose: bool = False) -> str:
    out = os.path.join(PKG, "libkldeval.so")
    tmp = out + ".tmp"
    cmd = compile_command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out
