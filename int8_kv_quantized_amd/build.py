"""Build libi8kv.so (HIP kernels + C ABI) for gfx950, in-tree."""
from __future__ import annotations

import os
import shutil
import subprocess
from pathlib import Path

HERE = Path(__file__).resolve().parent
CSRC = HERE / "csrc"
INCLUDE = HERE.parent / "include"
LIB = HERE / "libi8kv.so"
SOURCES = ["abi.hip", "producer.hip", "decode.hip", "prefill.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # IEEE fp32 division/sqrt and denormals: the producer's codes and scales
    # are bit-exact by definition.
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-gpu-flush-denormals-to-zero",
    "-fno-fast-math",
    # never emit packed fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and Path(cand).exists():
            return cand
    raise RuntimeError("hipcc not found")


def build(out: Path = LIB, extra=()) -> Path:
    out = Path(out)
    tmp = out.with_suffix(out.suffix + f".tmp{os.getpid()}")
    cmd = [hipcc(), *HIPCC_FLAGS, f"-I{INCLUDE}", *extra, *[str(CSRC / s) for s in SOURCES],
           "-o", str(tmp)]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
