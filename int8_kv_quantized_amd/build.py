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


# A checked build for the host side: the argument checks, plans and launch
# code compiled with AddressSanitizer and UndefinedBehaviorSanitizer (each
# flag applies to the host compilation only; the gfx950 kernels are built as
# usual).  It is loaded on the CPU, where no kernel runs, in a process that
# has the sanitizer runtime preloaded (sanitizer_env()).
SANITIZE_HOST = ["-g", "-Xarch_host", "-fsanitize=address,undefined",
                 "-Xarch_host", "-fno-sanitize-recover=all",
                 "-Xarch_host", "-fno-omit-frame-pointer"]
LIB_SANITIZED = HERE / "libi8kv_sanitized.so"


def sanitizer_env(env=None):
    """Environment for a child process that loads LIB_SANITIZED."""
    env = dict(os.environ if env is None else env)
    clang = Path(hipcc()).resolve().parent.parent / "llvm" / "bin" / "clang"
    if not clang.exists():
        clang = Path("/opt/rocm/llvm/bin/clang")
    rt = subprocess.run([str(clang), "-print-file-name=libclang_rt.asan-x86_64.so"], check=True,
                        capture_output=True, text=True).stdout.strip()
    env["LD_PRELOAD"] = rt
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    return env


def build(out: Path = LIB, extra=(), sanitize: bool = False) -> Path:
    out = Path(out)
    if sanitize:
        extra = [*SANITIZE_HOST, *extra]
        if out == LIB:
            out = LIB_SANITIZED
    tmp = out.with_suffix(out.suffix + f".tmp{os.getpid()}")
    cmd = [hipcc(), *HIPCC_FLAGS, f"-I{INCLUDE}", *extra, *[str(CSRC / s) for s in SOURCES],
           "-o", str(tmp)]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
