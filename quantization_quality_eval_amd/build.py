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
    return os.path.join(PKG, "libkldeval.so")


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


def build_library(verbose: bool = False) -> str:
    out = library_path()
    tmp = out + ".tmp"
    cmd = compile_command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out
