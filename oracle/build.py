"""Build step for the C oracle (test infrastructure; see oracle/__init__.py)."""
from __future__ import annotations

import os
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))


def oracle_library_path() -> str:
    return os.path.join(_HERE, "libkldoracle.so")


def build_oracle(verbose: bool = False) -> str:
    """Compile kld_oracle.c with gcc into oracle/libkldoracle.so.

    Portable x86-64 code (no -march=native): the library is built on one host
    and may run on another.
    """
    src = os.path.join(_HERE, "kld_oracle.c")
    out = oracle_library_path()
    tmp = out + ".tmp"
    cmd = ["gcc", "-O3", "-fPIC", "-shared", "-fopenmp", "-std=c11",
           "-Wall", "-Wextra", "-o", tmp, src, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out
