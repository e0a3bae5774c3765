"""Host-side tests of the C ABI (no GPU needed, nothing is launched).

* libi8kv.so loads and exports every function include/i8kv.h declares;
* every argument check returns its documented status before any launch
  (all calls below fail validation, so no kernel is ever enqueued).
"""
import ctypes as C
import re
from pathlib import Path

import pytest

import int8_kv_quantized_amd as K

ROOT = Path(__file__).resolve().parent.parent
HEADER = ROOT / "include" / "i8kv.h"
OK, NULL, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3, 4
FAKE = 0x100000  # 16-byte aligned stand-in pointer, never dereferenced


def declared_functions():
    text = re.sub(r"/\*.*?\*/", "", HEADER.read_text(), flags=re.S)
    return sorted(set(re.findall(r"\b(i8kv_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_operations():
    names = declared_functions()
    for op in ("i8kv_kv_quantize_write", "i8kv_kv_quantize_write_rope", "i8kv_paged_decode_int8",
               "i8kv_paged_decode_bf16pv", "i8kv_paged_decode_uint8w", "i8kv_paged_decode_ex",
               "i8kv_prefix_prefill_int8", "i8kv_prefix_prefill_bf16pv", "i8kv_decode_step_int8",
               "i8kv_paged_decode_bf16qk", "i8kv_prefix_prefill_bf16qk",
               "i8kv_paged_decode_partials", "i8kv_paged_decode_merge",
               "i8kv_prefix_prefill_uint8w", "i8kv_paged_decode_int8_noalloc",
               "i8kv_prefix_prefill_ex"):
        assert op in names


def test_library_exports_every_declared_symbol():
    lib = C.CDLL(str(K.lib_path()))
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, f"not exported: {missing}"


def test_abi_version_and_status_strings():
    assert K.abi_version() == 1
    for st in range(6):
        assert K.status_string(st)
    assert K.status_string(99) == "unknown status"


def _lib():
    return K.load_library()


def desc(Hq=24, Hkv=4, D=256, nb=64, bs=16):
    return K.CacheDesc(Hq, Hkv, D, nb, bs)


def producer(d, T=4, key=FAKE, value=FAKE, query=None, q8=None, qs=None, slot=FAKE,
             kc=FAKE, vc=FAKE, ks=FAKE, vs=FAKE):
    P = lambda x: None if x is None else C.c_void_p(x)
    return _lib().i8kv_kv_quantize_write(None if d is None else C.byref(d), T, P(key), P(value),
                                        P(query), P(q8), P(qs), P(slot), P(kc), P(vc), P(ks),
                                        P(vs), None)


def decode(d, S=1, max_len=512, max_blocks=32, part=256, G=32, ws=FAKE, ws_bytes=1 << 30,
           q8=FAKE, out=FAKE, scale=0.0625, bt=FAKE):
    P = lambda x: None if x is None else C.c_void_p(x)
    return _lib().i8kv_paged_decode_int8(
        None if d is None else C.byref(d), S, P(q8), P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE),
        P(bt), max_blocks, P(FAKE), max_len, part, G, scale, P(ws), ws_bytes, P(out), None)


def prefill(d, S=1, Tq=8, max_q=8, G=32, q8=FAKE, qsl=FAKE, scale=0.0625):
    P = lambda x: None if x is None else C.c_void_p(x)
    return _lib().i8kv_prefix_prefill_int8(
        None if d is None else C.byref(d), S, Tq, max_q, P(q8), P(FAKE), P(qsl), P(FAKE),
        P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE), 32, G, scale, None, 0, P(FAKE), None)


# --- producer ---------------------------------------------------------------
@pytest.mark.parametrize("kw,expect", [
    (dict(key=None), NULL), (dict(value=None), NULL), (dict(slot=None), NULL),
    (dict(kc=None), NULL), (dict(vs=None), NULL),
    (dict(query=FAKE, q8=None, qs=FAKE), NULL), (dict(query=FAKE, q8=FAKE, qs=None), NULL),
    (dict(T=-1), INVALID), (dict(key=FAKE + 2), INVALID), (dict(kc=FAKE + 8), INVALID),
    (dict(T=0), OK),
])
def test_producer_validation(kw, expect):
    assert producer(desc(), **kw) == expect


@pytest.mark.parametrize("d,expect", [
    (None, NULL), (desc(D=100), UNSUPPORTED), (desc(D=512), UNSUPPORTED),
    (desc(bs=32), UNSUPPORTED), (desc(Hq=24, Hkv=5), UNSUPPORTED),
    (desc(Hq=34, Hkv=2), UNSUPPORTED), (desc(Hq=0), INVALID), (desc(nb=0), INVALID),
])
def test_descriptor_validation(d, expect):
    assert producer(d) == expect
    assert decode(d) == expect
    assert prefill(d) == expect


def producer_rope(d, T=4, pos=FAKE, cs=FAKE, R=64, P_max=4096, **kw):
    P = lambda x: None if x is None else C.c_void_p(x)
    a = dict(key=FAKE, value=FAKE, query=None, q8=None, qs=None, slot=FAKE, kc=FAKE, vc=FAKE,
             ks=FAKE, vs=FAKE)
    a.update(kw)
    return _lib().i8kv_kv_quantize_write_rope(
        None if d is None else C.byref(d), T, P(a["key"]), P(a["value"]), P(a["query"]),
        P(a["q8"]), P(a["qs"]), P(a["slot"]), P(pos), P(cs), R, P_max, P(a["kc"]), P(a["vc"]),
        P(a["ks"]), P(a["vs"]), None)


@pytest.mark.parametrize("D,kw,expect", [
    (256, dict(pos=None), NULL), (256, dict(cs=None), NULL), (256, dict(key=None), NULL),
    (256, dict(query=FAKE, q8=None, qs=FAKE), NULL),
    (256, dict(P_max=0), INVALID), (256, dict(R=0), INVALID), (256, dict(cs=FAKE + 2), INVALID),
    (256, dict(T=-1), INVALID),
    (256, dict(R=260), UNSUPPORTED), (256, dict(R=68), UNSUPPORTED), (256, dict(R=3), UNSUPPORTED),
    (128, dict(R=66), UNSUPPORTED), (64, dict(R=33), UNSUPPORTED),
    (256, dict(R=72, T=0), OK), (256, dict(R=256, T=0), OK), (128, dict(R=4, T=0), OK),
    (64, dict(R=2, T=0), OK), (64, dict(R=64, T=0, cs=FAKE + 4), OK),
])
def test_producer_rope_validation(D, kw, expect):
    assert producer_rope(desc(D=D), **kw) == expect


def test_producer_rope_descriptor_checked():
    assert producer_rope(None) == NULL
    assert producer_rope(desc(D=100)) == UNSUPPORTED


# --- decode -------------------------------------------------------------------
def test_decode_workspace_query():
    d = desc()
    small = K.paged_decode_workspace_bytes(d, 1, 512)
    big = K.paged_decode_workspace_bytes(d, 16, 32768)
    assert 0 < small < big
    assert K.paged_decode_workspace_bytes(d, 1, 512, partition_size=512) == 0
    assert K.paged_decode_workspace_bytes(d, -1, 512) == 0


@pytest.mark.parametrize("kw,expect", [
    (dict(S=-1), INVALID), (dict(max_len=-1), INVALID), (dict(max_blocks=0), INVALID),
    (dict(max_len=16 * 32 + 1), INVALID), (dict(scale=float("nan")), INVALID),
    (dict(part=512), UNSUPPORTED), (dict(G=48), UNSUPPORTED), (dict(G=16), UNSUPPORTED),
    (dict(max_len=(1 << 20) + 16, max_blocks=1 << 17), UNSUPPORTED),
    (dict(q8=None), NULL), (dict(bt=None), NULL), (dict(out=None), NULL),
    (dict(q8=FAKE + 4), INVALID), (dict(out=FAKE + 4), INVALID),
    (dict(ws=None), WORKSPACE), (dict(ws_bytes=16), WORKSPACE), (dict(ws=FAKE + 16), WORKSPACE),
    (dict(S=0), OK),
])
def test_decode_validation(kw, expect):
    assert decode(desc(), **kw) == expect


def decode_partials(d, S=1, max_len=512, max_blocks=32, part=256, G=32, ws=FAKE,
                    ws_bytes=1 << 30, q8=FAKE, bt=FAKE, kc=FAKE, scale=0.0625):
    P = lambda x: None if x is None else C.c_void_p(x)
    return _lib().i8kv_paged_decode_partials(
        None if d is None else C.byref(d), S, P(q8), P(FAKE), P(kc), P(FAKE), P(FAKE), P(FAKE),
        P(bt), max_blocks, P(FAKE), max_len, part, G, scale, P(ws), ws_bytes, None)


def decode_merge(d, S=1, max_len=512, part=256, sl=FAKE, ws=FAKE, ws_bytes=1 << 30, out=FAKE):
    P = lambda x: None if x is None else C.c_void_p(x)
    return _lib().i8kv_paged_decode_merge(None if d is None else C.byref(d), S, P(sl), max_len,
                                         part, P(ws), ws_bytes, P(out), None)


@pytest.mark.parametrize("kw,expect", [
    (dict(q8=None), NULL), (dict(bt=None), NULL), (dict(kc=None), NULL),
    (dict(kc=FAKE + 4), INVALID), (dict(S=-1), INVALID), (dict(max_len=513), INVALID),
    (dict(scale=float("nan")), INVALID), (dict(part=512), UNSUPPORTED), (dict(G=16), UNSUPPORTED),
    (dict(ws=None), WORKSPACE), (dict(ws_bytes=16), WORKSPACE), (dict(ws=FAKE + 16), WORKSPACE),
    (dict(S=0), OK),
])
def test_decode_partials_validation(kw, expect):
    """The partials stage takes no output pointer; everything else as the call."""
    assert decode_partials(desc(), **kw) == expect
    assert decode_partials(None) == NULL
    assert decode_partials(desc(D=100)) == UNSUPPORTED


@pytest.mark.parametrize("kw,expect", [
    (dict(sl=None), NULL), (dict(out=None), NULL), (dict(out=FAKE + 4), INVALID),
    (dict(S=-1), INVALID), (dict(max_len=-1), INVALID), (dict(part=128), UNSUPPORTED),
    (dict(max_len=(1 << 20) + 1), UNSUPPORTED),
    (dict(ws=None), WORKSPACE), (dict(ws_bytes=16), WORKSPACE), (dict(ws=FAKE + 16), WORKSPACE),
    (dict(S=0), OK),
])
def test_decode_merge_validation(kw, expect):
    """The merge stage reads only the lengths and the workspace: no query,
    cache or block table is needed."""
    assert decode_merge(desc(), **kw) == expect
    assert decode_merge(None) == NULL
    assert decode_merge(desc(D=100)) == UNSUPPORTED


# --- fused decode step -----------------------------------------------------------
def decode_bf16pv(d, S=1, max_len=512, max_blocks=32, part=256, ws=FAKE, ws_bytes=1 << 30,
                  q8=FAKE, out=FAKE, scale=0.0625):
    P = lambda x: None if x is None else C.c_void_p(x)
    return _lib().i8kv_paged_decode_bf16pv(
        None if d is None else C.byref(d), S, P(q8), P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE),
        P(FAKE), max_blocks, P(FAKE), max_len, part, scale, P(ws), ws_bytes, P(out), None)


@pytest.mark.parametrize("kw,expect", [
    (dict(q8=None), NULL), (dict(out=None), NULL), (dict(S=-1), INVALID),
    (dict(max_len=513, max_blocks=32), INVALID), (dict(part=512), UNSUPPORTED),
    (dict(ws=None), WORKSPACE), (dict(ws_bytes=16), WORKSPACE), (dict(ws=FAKE + 16), WORKSPACE),
    (dict(scale=float("nan")), INVALID), (dict(S=0), OK),
])
def test_decode_bf16pv_validation(kw, expect):
    assert decode_bf16pv(desc(), **kw) == expect
    assert decode_bf16pv(None) == NULL
    assert decode_bf16pv(desc(D=100)) == UNSUPPORTED


def decode_uint8w(d, S=1, max_len=512, max_blocks=32, part=256, G=32, ws=FAKE,
                  ws_bytes=1 << 30, q8=FAKE, out=FAKE, scale=0.0625):
    P = lambda x: None if x is None else C.c_void_p(x)
    return _lib().i8kv_paged_decode_uint8w(
        None if d is None else C.byref(d), S, P(q8), P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE),
        P(FAKE), max_blocks, P(FAKE), max_len, part, G, scale, P(ws), ws_bytes, P(out), None)


@pytest.mark.parametrize("kw,expect", [
    (dict(q8=None), NULL), (dict(out=None), NULL), (dict(S=-1), INVALID),
    (dict(G=16), UNSUPPORTED), (dict(part=128), UNSUPPORTED), (dict(ws=None), WORKSPACE),
    (dict(ws_bytes=16), WORKSPACE), (dict(scale=float("inf")), INVALID), (dict(S=0), OK),
])
def test_decode_uint8w_validation(kw, expect):
    assert decode_uint8w(desc(), **kw) == expect
    assert decode_uint8w(None) == NULL


def decode_bf16qk(d, S=1, max_len=512, max_blocks=32, part=256, G=32, ws=FAKE,
                  ws_bytes=1 << 30, q=FAKE, out=FAKE, scale=0.0625):
    P = lambda x: None if x is None else C.c_void_p(x)
    return _lib().i8kv_paged_decode_bf16qk(
        None if d is None else C.byref(d), S, P(q), P(FAKE), P(FAKE), P(FAKE), P(FAKE),
        P(FAKE), max_blocks, P(FAKE), max_len, part, G, scale, P(ws), ws_bytes, P(out), None)


@pytest.mark.parametrize("kw,expect", [
    (dict(q=None), NULL), (dict(out=None), NULL), (dict(q=FAKE + 2), INVALID),
    (dict(S=-1), INVALID), (dict(max_len=513, max_blocks=32), INVALID), (dict(G=16), UNSUPPORTED),
    (dict(part=128), UNSUPPORTED), (dict(ws=None), WORKSPACE), (dict(ws_bytes=16), WORKSPACE),
    (dict(scale=float("inf")), INVALID), (dict(S=0), OK),
])
def test_decode_bf16qk_validation(kw, expect):
    assert decode_bf16qk(desc(), **kw) == expect
    assert decode_bf16qk(None) == NULL
    assert decode_bf16qk(desc(D=100)) == UNSUPPORTED


def decode_ex(d, opts_kw=None, S=1, max_len=512, max_blocks=32, ws=FAKE, ws_bytes=1 << 30,
              q8=FAKE, out=FAKE, no_opts=False):
    P = lambda x: None if x is None else C.c_void_p(x)
    o = dict(partition_size=256, w_group=32, softmax_scale=0.0625, pv=0, queries_per_seq=1,
             out_bf16=0)
    o.update(opts_kw or {})
    opts = K.DecodeOpts(**o)
    return _lib().i8kv_paged_decode_ex(
        None if d is None else C.byref(d), None if no_opts else C.byref(opts), S, P(q8), P(FAKE),
        P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE), max_blocks, P(FAKE), max_len, P(ws),
        ws_bytes, P(out), None)


@pytest.mark.parametrize("kw,expect", [
    (dict(no_opts=True), NULL), (dict(q8=None), NULL), (dict(out=None), NULL),
    (dict(opts_kw=dict(pv=3)), UNSUPPORTED), (dict(opts_kw=dict(out_bf16=2)), INVALID),
    (dict(opts_kw=dict(queries_per_seq=0)), INVALID),
    (dict(opts_kw=dict(queries_per_seq=3)), UNSUPPORTED),   # 3 * 6 rows > 16
    (dict(opts_kw=dict(queries_per_seq=2, w_group=48)), UNSUPPORTED),
    (dict(opts_kw=dict(queries_per_seq=2), ws_bytes=16), WORKSPACE),
    (dict(S=0, opts_kw=dict(queries_per_seq=2, pv=2, out_bf16=1)), OK),
    (dict(S=0, opts_kw=dict(pv=1, w_group=7)), OK),          # w_group unused by the bf16 PV
])
def test_decode_ex_validation(kw, expect):
    assert decode_ex(desc(), **kw) == expect


def test_decode_ex_workspace_query():
    o = dict(partition_size=256, w_group=32, softmax_scale=0.0625, pv=0, queries_per_seq=2,
             out_bf16=0)
    d = desc()
    ws = _lib().i8kv_paged_decode_ex_workspace_bytes
    one = ws(C.byref(d), C.byref(K.DecodeOpts(**dict(o, queries_per_seq=1))), 3, 4096)
    two = ws(C.byref(d), C.byref(K.DecodeOpts(**o)), 3, 4096)
    assert one == K.paged_decode_workspace_bytes(d, 3, 4096) and two > one
    assert _lib().i8kv_paged_decode_ex_workspace_bytes(C.byref(d), None, 3, 4096) == 0


def decode_step(d, S=2, key=FAKE, value=FAKE, query=FAKE, q8=None, qs=None, kc=FAKE, vc=FAKE,
                ks=FAKE, vs=FAKE, bt=FAKE, max_blocks=32, sl=FAKE, max_len=512, part=256, G=32,
                scale=0.0625, ws=FAKE, ws_bytes=1 << 30, out=FAKE):
    P = lambda x: None if x is None else C.c_void_p(x)
    return _lib().i8kv_decode_step_int8(
        None if d is None else C.byref(d), S, P(key), P(value), P(query), P(q8), P(qs), P(kc),
        P(vc), P(ks), P(vs), P(bt), max_blocks, P(sl), max_len, part, G, scale, P(ws), ws_bytes,
        P(out), None)


@pytest.mark.parametrize("kw,expect", [
    (dict(key=None), NULL), (dict(value=None), NULL), (dict(query=None), NULL),
    (dict(q8=FAKE), NULL), (dict(qs=FAKE), NULL), (dict(kc=None), NULL), (dict(out=None), NULL),
    (dict(key=FAKE + 2), INVALID), (dict(q8=FAKE + 4, qs=FAKE), INVALID),
    (dict(S=-1), INVALID), (dict(max_len=16 * 32 + 1), INVALID), (dict(G=16), UNSUPPORTED),
    (dict(part=128), UNSUPPORTED), (dict(ws=None), WORKSPACE), (dict(ws_bytes=16), WORKSPACE),
    (dict(S=0), OK), (dict(S=0, q8=FAKE, qs=FAKE), OK),
])
def test_decode_step_validation(kw, expect):
    assert decode_step(desc(), **kw) == expect


def test_decode_step_descriptor_checked_first():
    assert decode_step(None) == NULL
    assert decode_step(desc(D=96)) == UNSUPPORTED


# --- prefill ------------------------------------------------------------------
def prefill_ex(d, opts_kw=None, S=1, Tq=8, max_q=8, q8=FAKE, out=FAKE, no_opts=False):
    P = lambda x: None if x is None else C.c_void_p(x)
    o = dict(w_group=32, softmax_scale=0.0625, pv=0, out_bf16=0)
    o.update(opts_kw or {})
    opts = K.PrefillOpts(**o)
    return _lib().i8kv_prefix_prefill_ex(
        None if d is None else C.byref(d), None if no_opts else C.byref(opts), S, Tq, max_q,
        P(q8), P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE), 32, P(out),
        None)


@pytest.mark.parametrize("kw,expect", [
    (dict(no_opts=True), NULL), (dict(q8=None), NULL), (dict(out=None), NULL),
    (dict(opts_kw=dict(pv=3)), UNSUPPORTED), (dict(opts_kw=dict(out_bf16=2)), INVALID),
    (dict(opts_kw=dict(w_group=48)), UNSUPPORTED),
    (dict(opts_kw=dict(out_bf16=1), out=FAKE + 4), INVALID),   # bf16 out: 8-byte aligned
    (dict(opts_kw=dict(out_bf16=1), out=FAKE + 8, S=0), OK),
    (dict(S=0, opts_kw=dict(pv=1, w_group=7)), OK),           # w_group unused by the bf16 PV
    (dict(S=0, opts_kw=dict(pv=2, out_bf16=1)), OK),
    (dict(S=-1), INVALID),
])
def test_prefill_ex_validation(kw, expect):
    assert prefill_ex(desc(), **kw) == expect
    assert prefill_ex(None) == NULL



@pytest.mark.parametrize("kw,expect", [
    (dict(S=-1), INVALID), (dict(Tq=-1), INVALID), (dict(max_q=9), INVALID),
    (dict(G=16), UNSUPPORTED), (dict(scale=float("inf")), INVALID),
    (dict(q8=None), NULL), (dict(qsl=None), NULL), (dict(q8=FAKE + 1), INVALID),
    (dict(S=0), OK), (dict(Tq=0, max_q=0), OK),
])
def test_prefill_validation(kw, expect):
    assert prefill(desc(), **kw) == expect


def prefill_bf16qk(d, S=1, Tq=8, max_q=8, G=32, q=FAKE, qsl=FAKE, scale=0.0625):
    P = lambda x: None if x is None else C.c_void_p(x)
    return _lib().i8kv_prefix_prefill_bf16qk(
        None if d is None else C.byref(d), S, Tq, max_q, P(q), P(qsl), P(FAKE), P(FAKE),
        P(FAKE), P(FAKE), P(FAKE), P(FAKE), 32, G, scale, None, 0, P(FAKE), None)


@pytest.mark.parametrize("kw,expect", [
    (dict(S=-1), INVALID), (dict(Tq=-1), INVALID), (dict(max_q=9), INVALID),
    (dict(G=16), UNSUPPORTED), (dict(scale=float("nan")), INVALID),
    (dict(q=None), NULL), (dict(qsl=None), NULL), (dict(q=FAKE + 2), INVALID),
    (dict(S=0), OK), (dict(Tq=0, max_q=0), OK),
])
def test_prefill_bf16qk_validation(kw, expect):
    assert prefill_bf16qk(desc(), **kw) == expect
    assert prefill_bf16qk(None) == NULL
    assert prefill_bf16qk(desc(D=100)) == UNSUPPORTED


def test_binding_rejects_missing_library(monkeypatch, tmp_path):
    from int8_kv_quantized_amd import _binding
    monkeypatch.setattr(_binding, "_lib", None)
    monkeypatch.setattr(_binding, "HERE", tmp_path)
    with pytest.raises(RuntimeError, match="no fallback"):
        _binding.load_library()


def test_loading_the_library_brings_torch_in_first():
    """The library must bind to torch's HIP runtime: loading it in a fresh
    process with nothing else imported also imports torch, before the dlopen."""
    import subprocess
    import sys
    code = ("import sys; sys.path.insert(0, %r); import int8_kv_quantized_amd as K; "
            "assert 'torch' not in sys.modules; K.load_library(); "
            "assert 'torch' in sys.modules; print('ok')" % str(ROOT))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stderr[-2000:]


def test_noalloc_decode_size_checks_before_any_device_call():
    """The no-allocation decode rejects a descriptor or a size past its fixed
    array before it asks the runtime for anything (no GPU is needed here)."""
    P = C.c_void_p
    lib = _lib()
    assert lib.i8kv_paged_decode_noalloc_max_bytes() == 64 << 20
    d = desc()
    args = lambda dd, S, L: (None if dd is None else C.byref(dd), S, P(FAKE), P(FAKE), P(FAKE),
                             P(FAKE), P(FAKE), P(FAKE), P(FAKE), max(1, L // 16), P(FAKE), L, 256,
                             32, 0.0625, P(FAKE), None)
    assert lib.i8kv_paged_decode_int8_noalloc(*args(None, 1, 512)) == NULL
    assert lib.i8kv_paged_decode_int8_noalloc(*args(desc(D=100), 1, 512)) == UNSUPPORTED
    assert K.paged_decode_workspace_bytes(d, 32, 32768) > 64 << 20
    assert lib.i8kv_paged_decode_int8_noalloc(*args(d, 32, 32768)) == WORKSPACE
    assert K.paged_decode_workspace_bytes(d, 16, 32768) <= 64 << 20


def test_prefill_uint8w_validation():
    """The UINT8-W prefill validates as the int8 prefill does, before any launch."""
    P = lambda x: None if x is None else C.c_void_p(x)
    lib = _lib()

    def call(d, S=1, Tq=8, max_q=8, G=32, q8=FAKE, qsl=FAKE, scale=0.0625):
        return lib.i8kv_prefix_prefill_uint8w(
            None if d is None else C.byref(d), S, Tq, max_q, P(q8), P(FAKE), P(qsl), P(FAKE),
            P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE), 32, G, scale, None, 0, P(FAKE), None)
    assert call(None) == NULL
    assert call(desc(D=100)) == UNSUPPORTED
    assert call(desc(), q8=None) == NULL
    assert call(desc(), qsl=None) == NULL
    assert call(desc(), G=48) == UNSUPPORTED
    assert call(desc(), S=-1) == INVALID
    assert call(desc(), max_q=9) == INVALID
    assert call(desc(), scale=float("inf")) == INVALID
    assert call(desc(), q8=FAKE + 4) == INVALID
    assert call(desc(), S=0) == OK
