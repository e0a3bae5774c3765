"""Build the C++ oracle into a shared library (test infrastructure).

The oracle is compiled with plain ``g++ -O2`` and IEEE semantics: no
fast-math, no FP contraction, denormals kept.
"""
from __future__ import annotations

import os
import subprocess
import sys
from pathlib import Path

HERE = Path(__file__).resolve().parent
SRC = HERE / "oracle.cpp"
LIB = HERE / "liboracle.so"

CXXFLAGS = ["-O2", "-std=c++17", "-fPIC", "-shared", "-fno-fast-math",
            "-ffp-contract=off", "-fno-finite-math-only", "-Wall", "-Wextra"]


# A checked CPU build: AddressSanitizer (out-of-bounds reads and writes of the
# caches, tables and traces) and UndefinedBehaviorSanitizer (signed overflow,
# bad shifts, invalid casts) abort on the first finding.  A process that
# loads it needs the sanitizer runtime preloaded (sanitizer_env()).
SANITIZE = ["-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
            "-fno-sanitize-recover=all"]
LIB_SANITIZED = HERE / "liboracle_sanitized.so"


def sanitizer_env(env=None):
    """Environment for a child process that loads a sanitized build."""
    env = dict(os.environ if env is None else env)
    rt = subprocess.run(["g++", "-print-file-name=libasan.so"], check=True, capture_output=True,
                        text=True).stdout.strip()
    env["LD_PRELOAD"] = rt
    # the interpreter itself is not instrumented: its own allocations are not
    # leaks of the oracle
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:strict_string_checks=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    return env


def build(src: Path = SRC, out: Path = LIB, extra=(), sanitize: bool = False) -> Path:
    src, out = Path(src), Path(out)
    if sanitize:
        extra = [*SANITIZE, *extra]
    out.parent.mkdir(parents=True, exist_ok=True)
    tmp = out.with_suffix(out.suffix + f".tmp{os.getpid()}")
    cmd = ["g++", *CXXFLAGS, f"-I{HERE}", *extra, str(src), "-o", str(tmp)]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
    sys.exit(0)
