"""Build step for the C oracle (test infrastructure; see oracle/__init__.py)."""
from __future__ import annotations

import os
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))


def oracle_library_path() -> str:
    """The in-tree library, or the build named by KLD_ORACLE_LIBRARY."""
    return os.environ.get("KLD_ORACLE_LIBRARY") or os.path.join(_HERE, "libkldoracle.so")


def build_oracle(verbose: bool = False, native: bool = False, out: str | None = None) -> str:
    """Compile kld_oracle.c with gcc into oracle/libkldoracle.so (or ``out``).

    By default portable x86-64 code: the in-tree library is built on one host
    and may run on another. ``native`` adds -march=native, for a copy compiled
    and timed on the host that runs it (the benchmark's CPU baseline).
    """
    src = os.path.join(_HERE, "kld_oracle.c")
    out = out or os.path.join(_HERE, "libkldoracle.so")
    tmp = out + ".tmp"
    cmd = ["gcc", "-O3", *(["-march=native"] if native else []), "-fPIC", "-shared", "-fopenmp", "-std=c11",
           "-Wall", "-Wextra", "-o", tmp, src, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build_sanitized_oracle(out: str, clang: str = "/opt/rocm/llvm/bin/clang", verbose: bool = False) -> str:
    """kld_oracle.c with AddressSanitizer and UndefinedBehaviorSanitizer, built
    by clang so that it shares one sanitizer runtime with the host code of the
    HIP library's sanitizer build (hipcc's host compiler is the same clang)."""
    src = os.path.join(_HERE, "kld_oracle.c")
    tmp = out + ".tmp"
    cmd = [clang, "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-fPIC", "-shared", "-fopenmp", "-std=c11",
           "-Wall", "-Wextra", "-o", tmp, src, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out
