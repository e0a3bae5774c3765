"""Host-side logic of bench.py (CPU only): the one-GPU rule and the lookup of
the committed HBM-traffic counters."""
import json
import shutil
import subprocess
import sys
from pathlib import Path

import bench

ROOT = Path(__file__).resolve().parents[1]


def test_more_than_one_gpu_is_refused_before_any_device_work():
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""          # no JSON line for a refused run


def test_importing_bench_loads_neither_the_oracle_nor_the_library():
    code = ("import sys; sys.path.insert(0, %r); import bench; "
            "print(any(m == 'oracle' or m.startswith('oracle.') for m in sys.modules), "
            "'int8_kv_quantized_amd' in sys.modules)" % str(ROOT))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    assert r.stdout.split() == ["False", "False"]


def _tree_with(tmp_path, records, edit_source=False, edited=None):
    """A copy of the files counted_traffic reads, under tmp_path."""
    for s in dict.fromkeys(bench.DECODE_SOURCES + bench.PREFILL_SOURCES):
        dst = tmp_path / s
        dst.parent.mkdir(parents=True, exist_ok=True)
        shutil.copy(ROOT / s, dst)
    if edit_source:
        p = tmp_path / (edited or bench.DECODE_SOURCES[0])
        p.write_text(p.read_text() + "\n// edited\n")
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / "hbm_traffic.json").write_text(json.dumps(records))


def test_traffic_is_the_committed_per_launch_bytes_of_the_partition_kernel():
    """The committed record's bytes while the hashed sources are those it was
    taken on, null otherwise (a stale count is never reported)."""
    import hashlib
    recs = json.loads((ROOT / "profiles" / "hbm_traffic.json").read_text())
    rec = [r for r in recs if r["workload"] == "decode_L16384_outlierV_G32" and r["w_group"] == 32][0]
    h = hashlib.sha256()
    for src in bench.DECODE_SOURCES:
        h.update((ROOT / src).read_bytes())
    want = rec["hbm_bytes_per_launch"] if h.hexdigest() == rec["kernel_sources_sha256"] else None
    assert bench.counted_traffic("decode_L16384_outlierV_G32", 32) == want
    # the partition kernel moves at least the algorithmic K/V + scale bytes
    assert rec["hbm_bytes_per_launch"] >= 34078720
    assert bench.counted_traffic("decode_L16384_outlierV_G32", 64) is None
    assert bench.counted_traffic("decode_L512", 32) is None


def _rehashed(recs):
    """The committed records, keyed to the current decode sources."""
    import hashlib
    h = hashlib.sha256()
    for src in bench.DECODE_SOURCES:
        h.update((ROOT / src).read_bytes())
    return [dict(r, kernel_sources_sha256=h.hexdigest()) for r in recs]


def test_traffic_is_null_once_a_decode_source_changes(tmp_path, monkeypatch):
    recs = _rehashed(json.loads((ROOT / "profiles" / "hbm_traffic.json").read_text()))
    _tree_with(tmp_path, recs)
    monkeypatch.setattr(bench, "ROOT", tmp_path)
    assert bench.counted_traffic("decode_L16384_outlierV_G32", 32) is not None
    _tree_with(tmp_path / "edited", recs, edit_source=True)
    monkeypatch.setattr(bench, "ROOT", tmp_path / "edited")
    assert bench.counted_traffic("decode_L16384_outlierV_G32", 32) is None


def test_traffic_needs_a_per_launch_record(tmp_path, monkeypatch):
    recs = _rehashed(json.loads((ROOT / "profiles" / "hbm_traffic.json").read_text()))
    for r in recs:
        r.pop("hbm_bytes_per_launch")   # a call-level record is not a launch's traffic
    _tree_with(tmp_path, recs)
    monkeypatch.setattr(bench, "ROOT", tmp_path)
    assert bench.counted_traffic("decode_L16384_outlierV_G32", 32) is None


def _sha(sources):
    import hashlib
    h = hashlib.sha256()
    for src in sources:
        h.update((ROOT / src).read_bytes())
    return h.hexdigest()


def test_prefill_traffic_is_the_committed_per_launch_bytes_of_the_prefill_kernel():
    """The prefill records are keyed to the prefill kernel's sources: their
    bytes while those are unchanged, null otherwise, and never returned for
    the decode's sources or another W group."""
    recs = json.loads((ROOT / "profiles" / "hbm_traffic.json").read_text())
    fresh = _sha(bench.PREFILL_SOURCES)
    for G in (32, 64):
        name = f"prefill_2048_over_16384_G{G}"
        rec = [r for r in recs if r["workload"] == name and r["w_group"] == G][0]
        want = rec["hbm_bytes_per_launch"] if rec["kernel_sources_sha256"] == fresh else None
        assert bench.counted_traffic(name, G, bench.PREFILL_SOURCES) == want
        # at least one pass over K/V and scales (38.3 MB), the int8 queries and
        # their scales (12.8 MB) and the fp32 output (50.3 MB)
        assert rec["hbm_bytes_per_launch"] >= 38_338_560 + 12_779_520 + 50_331_648
        assert bench.counted_traffic(name, G) is None            # decode sources
        assert bench.counted_traffic(name, 96 - G, bench.PREFILL_SOURCES) is None


def test_prefill_traffic_is_null_once_a_prefill_source_changes(tmp_path, monkeypatch):
    recs = json.loads((ROOT / "profiles" / "hbm_traffic.json").read_text())
    fresh = _sha(bench.PREFILL_SOURCES)
    recs = [dict(r, kernel_sources_sha256=fresh) if r["workload"].startswith("prefill_") else r
            for r in recs]
    name = "prefill_2048_over_16384_G32"
    _tree_with(tmp_path, recs)
    monkeypatch.setattr(bench, "ROOT", tmp_path)
    assert bench.counted_traffic(name, 32, bench.PREFILL_SOURCES) is not None
    _tree_with(tmp_path / "edited", recs, edit_source=True, edited=bench.PREFILL_SOURCES[0])
    monkeypatch.setattr(bench, "ROOT", tmp_path / "edited")
    assert bench.counted_traffic(name, 32, bench.PREFILL_SOURCES) is None
