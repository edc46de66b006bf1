"""Host-side sanitizer run of the CPU test suite.

Builds the HIP library with its host code (argument validation, handle
registry, events, workspace growth, the C ABI's error paths) under
AddressSanitizer and UndefinedBehaviorSanitizer, and the C oracle the same
way, as separate files under _build/sanitize/ (the normal builds are left
alone), then runs ``pytest -m "not gpu"`` against them with clang's ASan
runtime preloaded. Any sanitizer report aborts the run.

Run from the repository root:   python tests/run_sanitized.py [pytest args]
(default: tests -m "not gpu" -q). Needs no GPU.
"""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from oracle.build import build_sanitized_oracle  # noqa: E402
from quantization_quality_eval_amd.build import build_sanitized_library  # noqa: E402

CLANG = "/opt/rocm/llvm/bin/clang"


def main() -> int:
    out = os.path.join(ROOT, "_build", "sanitize")
    os.makedirs(out, exist_ok=True)
    lib = build_sanitized_library(os.path.join(out, "libkldeval_asan.so"))
    orc = build_sanitized_oracle(os.path.join(out, "libkldoracle_asan.so"), clang=CLANG)
    runtime = subprocess.run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True,
                             check=True).stdout.strip()
    llvm_lib = os.path.join(os.path.dirname(os.path.dirname(CLANG)), "lib")
    env = dict(os.environ,
               LD_PRELOAD=runtime,
               LD_LIBRARY_PATH=os.pathsep.join(p for p in (llvm_lib, os.environ.get("LD_LIBRARY_PATH")) if p),
               # Python and the libraries it loads keep allocations alive until exit by design
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1:detect_odr_violation=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1",
               KLD_EVAL_LIBRARY=lib, KLD_ORACLE_LIBRARY=orc, KLD_SANITIZED="1")
    args = sys.argv[1:] or ["tests", "-m", "not gpu", "-q", "-p", "no:cacheprovider"]
    print(f"[sanitize] {lib}\n[sanitize] {orc}\n[sanitize] pytest {' '.join(args)}", flush=True)
    return subprocess.call([sys.executable, "-m", "pytest", *args], env=env, cwd=ROOT)


if __name__ == "__main__":
    sys.exit(main())
