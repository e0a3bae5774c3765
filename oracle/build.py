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


def build(src: Path = SRC, out: Path = LIB, extra=()) -> Path:
    src, out = Path(src), Path(out)
    out.parent.mkdir(parents=True, exist_ok=True)
    tmp = out.with_suffix(out.suffix + f".tmp{os.getpid()}")
    cmd = ["g++", *CXXFLAGS, f"-I{HERE}", *extra, str(src), "-o", str(tmp)]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
    sys.exit(0)
