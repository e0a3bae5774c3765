"""The oracle's pins, and planted mistakes that move indices and layouts,
under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

A checked build of oracle/oracle.cpp is loaded in a child process with the
sanitizer runtime preloaded; every pin must pass there with no sanitizer
report (a report aborts the child), and the index-moving mutants must still
be caught by a pin without reading or writing out of bounds.  Fast code can
be wrong code, as the INT8 KV page's section 5.4 notes; these runs show the
checker itself reads only what it should.
"""
import subprocess
import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parent.parent

# mutants that change an index, a layout or a loop bound
INDEX_MUTANTS = ["k_layout_token_major", "v_layout_dim_inner", "scale_layout_head_major",
                 "page_offset_shift", "gqa_modulo", "misgrouped_w_scale", "prefill_not_causal",
                 "prefill_excludes_self", "rope_interleaved_pairs", "rope_position_off_by_one",
                 "bf16qk_dims_reversed", "bf16qk_first_head_query"]

CHILD = r'''
import sys, tempfile
from pathlib import Path
sys.path[:0] = [sys.argv[1], sys.argv[1] + "/tests"]
import pins
from oracle import Oracle, build as obuild
import test_oracle_mutants as M

lib = obuild.build(out=obuild.LIB_SANITIZED, sanitize=True, extra=["-w"])
orc = Oracle(lib)
for pin in pins.ALL_PINS:
    pin(orc)
for pin in (pins.pin_decode_trace, pins.pin_decode_bruteforce, pins.pin_decode_partition_invariance,
            pins.pin_prefill_trace, pins.pin_prefill_vs_decode):
    pin(orc, G=64)
print("pins ok", flush=True)
with tempfile.TemporaryDirectory() as tmp:
    for name in sys.argv[2:]:
        src = M.SRC.read_text()
        for old, new in M.MUTANTS[name]:
            assert src.count(old) >= 1, name
            src = src.replace(old, new)
        d = Path(tmp) / name
        d.mkdir()
        (d / "oracle.cpp").write_text(src)
        morc = Oracle(obuild.build(d / "oracle.cpp", d / "liboracle.so", extra=["-w"],
                                   sanitize=True))
        caught = []
        for pin in pins.ALL_PINS:
            try:
                pin(morc)
            except (AssertionError, ValueError, FloatingPointError, IndexError):
                caught.append(pin.__name__)
        assert caught, f"no pin caught {name}"
        print(f"{name}: caught by {len(caught)} pins", flush=True)
print("sanitized run ok", flush=True)
'''


@pytest.mark.slow
def test_pins_and_index_mutants_under_sanitizers():
    sys.path.insert(0, str(ROOT))
    from oracle import build as obuild
    r = subprocess.run([sys.executable, "-c", CHILD, str(ROOT), *INDEX_MUTANTS],
                       env=obuild.sanitizer_env(), capture_output=True, text=True, timeout=900)
    print(r.stdout[-3000:])
    assert r.returncode == 0, f"sanitized oracle run failed ({r.returncode}):\n{r.stderr[-4000:]}"
    assert "sanitized run ok" in r.stdout
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr


LIVE_CHECK = r'''
import sys, tempfile
from pathlib import Path
sys.path[:0] = [sys.argv[1], sys.argv[1] + "/tests"]
import pins
from oracle import Oracle, build as obuild
import test_oracle_mutants as M
src = M.SRC.read_text()
old = "int8_t kq(int i, int d) const { return c->k[c->k_index(page(i), kv, off(i), d)]; }"
assert src.count(old) == 1
# one page past the last one: outside the cache array
src = src.replace(old, "int8_t kq(int i, int d) const { return c->k[c->k_index(c->nb, kv, off(i), d)]; }")
with tempfile.TemporaryDirectory() as tmp:
    (Path(tmp) / "oracle.cpp").write_text(src)
    orc = Oracle(obuild.build(Path(tmp) / "oracle.cpp", Path(tmp) / "liboracle.so", extra=["-w"],
                              sanitize=True))
    pins.pin_decode_trace(orc)
print("no report", flush=True)
'''


@pytest.mark.slow
def test_sanitizer_reports_a_planted_out_of_bounds_read():
    """The checked build is live: a key read one page past the cache (planted
    on the CPU, in a copy of the oracle) aborts the child with a report."""
    sys.path.insert(0, str(ROOT))
    from oracle import build as obuild
    r = subprocess.run([sys.executable, "-c", LIVE_CHECK, str(ROOT)], env=obuild.sanitizer_env(),
                       capture_output=True, text=True, timeout=600)
    assert r.returncode != 0 and "no report" not in r.stdout
    assert "AddressSanitizer" in r.stderr, r.stderr[-2000:]
