"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only).

libi8kv.so is rebuilt with both sanitizers on its host compilation (argument
checks, workspace plans, launch code; the gfx950 kernels are compiled as
usual and never run here) and every host-side ABI test (tests/test_abi_host.py:
each documented status of every call, sizes, alignment, the workspace
queries) runs against it in a child process with the sanitizer runtime
preloaded; the first finding aborts the child.  (This is how an enum value
outside the status range, read in i8kv_status_string, was found: the call
now takes an int32_t.)"""
import subprocess
import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parent.parent

RUNNER = r"""
import sys
from pathlib import Path
sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r})
import atexit, os, shutil, tempfile
import int8_kv_quantized_amd._binding as B
# the package loads HERE / "libi8kv.so": point HERE at a folder whose
# libi8kv.so is the sanitized build (tests that move HERE still work)
d = tempfile.mkdtemp()
atexit.register(shutil.rmtree, d, True)
os.symlink(sys.argv[1], os.path.join(d, "libi8kv.so"))
B.HERE = Path(d)
import pytest
sys.exit(pytest.main(["-q", "-x", "-p", "no:cacheprovider", {abi!r}]))
"""


@pytest.fixture(scope="module")
def sanitized_lib():
    from int8_kv_quantized_amd import build
    return build.build(sanitize=True)


def test_sanitized_build_is_instrumented(sanitized_lib):
    syms = subprocess.run(["nm", "-D", "--undefined-only", str(sanitized_lib)], check=True,
                          capture_output=True, text=True).stdout
    assert "__asan_report_load" in syms, "no AddressSanitizer checks in the host code"
    assert "__ubsan_handle" in syms, "no UndefinedBehaviorSanitizer checks in the host code"


def test_abi_host_checks_under_sanitizers(sanitized_lib):
    from int8_kv_quantized_amd import build
    code = RUNNER.format(root=str(ROOT), tests=str(ROOT / "tests"),
                         abi=str(ROOT / "tests" / "test_abi_host.py"))
    r = subprocess.run([sys.executable, "-c", code, str(sanitized_lib)], capture_output=True,
                       text=True, timeout=900, env=build.sanitizer_env())
    tail = (r.stdout[-4000:] + "\n" + r.stderr[-4000:])
    assert r.returncode == 0, f"sanitized ABI tests failed (rc {r.returncode}):\n{tail}"
    assert " passed" in r.stdout
