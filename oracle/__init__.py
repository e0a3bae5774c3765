"""Python access to the C++ oracle -- TEST INFRASTRUCTURE ONLY.

The oracle (``oracle.cpp``) is the plain single-threaded CPU definition of
paged attention over an INT8 KV cache.  Only the tests, the package smoke
check and the benchmark's CPU-baseline leg may import this module; the
product path never does.  This wrapper only marshals numpy arrays.
"""
from __future__ import annotations

import ctypes as C
from pathlib import Path
from typing import Optional

import numpy as np

from . import build as _build

HERE = Path(__file__).resolve().parent
ORC_NO_WQUANT = 1
ORC_EXACT = 2
ORC_BF16_PV = 4
ORC_UINT8_W = 8

_P = C.c_void_p
_I = C.c_int
_F = C.c_float


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


class _DecodeTrace(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("s", "P", "W", "Wq", "sW", "m", "l", "o", "acc")]


class _PrefillTrace(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("s", "ptil", "Wq", "sW", "m_tile", "l")]


class Oracle:
    """ctypes view of one build of the oracle library."""

    def __init__(self, lib_path: Optional[Path] = None):
        if lib_path is None:
            lib_path = _build.LIB
            if not Path(lib_path).exists():
                _build.build()
        self.path = Path(lib_path)
        self.lib = C.CDLL(str(self.path))
        L = self.lib
        L.orc_expf.restype = C.c_float
        L.orc_expf.argtypes = [C.c_float]
        L.orc_quantize.restype = None
        L.orc_quantize.argtypes = [_P, _I, _P, _P]
        L.orc_quantize_w.restype = None
        L.orc_quantize_w.argtypes = [_P, _I, _P, _P]
        L.orc_quantize_w_u8.restype = None
        L.orc_quantize_w_u8.argtypes = [_P, _I, _P, _P]
        L.orc_kv_quantize_write.argtypes = [_I] * 6 + [_P] * 10
        L.orc_kv_quantize_write_rope.argtypes = [_I] * 6 + [_P] * 8 + [_I, _I] + [_P] * 4
        L.orc_rope_rotate.argtypes = [_I, _I, _P, _P, _P, _I, _I]
        L.orc_round_bf16.restype = None
        L.orc_round_bf16.argtypes = [_P, _I, _P]
        L.orc_paged_decode.argtypes = ([_I] * 6 + [_P] * 7 + [_I, _P, _I, _I, _F, _I, _P])
        L.orc_decode_head.argtypes = ([_I] * 7 + [_P] * 7 + [_I, _P, _I, _I, _F, _I,
                                                              C.POINTER(_DecodeTrace), _P])
        L.orc_prefix_prefill.argtypes = ([_I] * 7 + [_P] * 9 + [_I, _I, _I, _F, _I,
                                                                _P, _I, _P])
        L.orc_prefill_row.argtypes = ([_I] * 9 + [_P] * 9 + [_I, _I, _I, _F, _I,
                                                             C.POINTER(_PrefillTrace), _P])
        L.orc_paged_decode_bf16qk.argtypes = ([_I] * 6 + [_P] * 6 + [_I, _P, _I, _I, _F, _I,
                                                                     _P])
        L.orc_prefix_prefill_bf16qk.argtypes = ([_I] * 7 + [_P] * 8 + [_I, _I, _I, _F, _I,
                                                                       _P, _I, _P])

    # ------------------------------------------------------------------
    def expf(self, x: float) -> float:
        return float(self.lib.orc_expf(float(x)))

    def quantize(self, x: np.ndarray):
        x = _c(x, np.float32)
        q = np.zeros(x.shape, np.int8)
        s = np.zeros(1, np.float32)
        self.lib.orc_quantize(_ptr(x), x.size, _ptr(q), _ptr(s))
        return q, np.float32(s[0])

    def quantize_w(self, w: np.ndarray):
        w = _c(w, np.float32)
        q = np.zeros(w.shape, np.int8)
        s = np.zeros(1, np.float32)
        self.lib.orc_quantize_w(_ptr(w), w.size, _ptr(q), _ptr(s))
        return q, np.float32(s[0])

    def quantize_w_u8(self, w: np.ndarray):
        w = _c(w, np.float32)
        q = np.zeros(w.shape, np.uint8)
        s = np.zeros(1, np.float32)
        self.lib.orc_quantize_w_u8(_ptr(w), w.size, _ptr(q), _ptr(s))
        return q, np.float32(s[0])

    # ------------------------------------------------------------------
    @staticmethod
    def empty_cache(num_blocks, num_kv_heads, head_dim, block_size=16):
        nb, H, D, bs = num_blocks, num_kv_heads, head_dim, block_size
        return dict(k_cache=np.zeros((nb, H, D // 16, bs, 16), np.int8),
                    v_cache=np.zeros((nb, H, D, bs), np.int8),
                    k_scale=np.zeros((nb, bs, H), np.float32),
                    v_scale=np.zeros((nb, bs, H), np.float32))

    def kv_quantize_write(self, key, value, slot_mapping, cache, *, num_q_heads,
                          query=None):
        key = _c(key, np.uint16)
        value = _c(value, np.uint16)
        slot = _c(slot_mapping, np.int32)
        T, Hkv, D = key.shape
        nb, _, _, bs, _ = cache["k_cache"].shape
        q_int8 = q_scale = None
        if query is not None:
            query = _c(query, np.uint16)
            q_int8 = np.zeros(query.shape, np.int8)
            q_scale = np.zeros(query.shape[:2], np.float32)
        rc = self.lib.orc_kv_quantize_write(
            T, num_q_heads, Hkv, D, bs, nb, _ptr(key), _ptr(value), _ptr(query),
            _ptr(q_int8), _ptr(q_scale), _ptr(slot), _ptr(cache["k_cache"]),
            _ptr(cache["v_cache"]), _ptr(cache["k_scale"]), _ptr(cache["v_scale"]))
        if rc:
            raise ValueError(f"orc_kv_quantize_write rejected its arguments ({rc})")
        return q_int8, q_scale

    def kv_quantize_write_rope(self, key, value, slot_mapping, positions, cos_sin, cache, *,
                               num_q_heads, query=None):
        """The producer with RoPE on Q and K (rotate-half pairing over the
        first cos_sin.shape[1] dims, cos_sin [max_position, R] = cos | sin)."""
        key = _c(key, np.uint16)
        value = _c(value, np.uint16)
        slot = _c(slot_mapping, np.int32)
        pos = _c(positions, np.int32)
        cs = _c(cos_sin, np.float32)
        T, Hkv, D = key.shape
        nb, _, _, bs, _ = cache["k_cache"].shape
        q_int8 = q_scale = None
        if query is not None:
            query = _c(query, np.uint16)
            q_int8 = np.zeros(query.shape, np.int8)
            q_scale = np.zeros(query.shape[:2], np.float32)
        rc = self.lib.orc_kv_quantize_write_rope(
            T, num_q_heads, Hkv, D, bs, nb, _ptr(key), _ptr(value), _ptr(query),
            _ptr(q_int8), _ptr(q_scale), _ptr(slot), _ptr(pos), _ptr(cs), cs.shape[1],
            cs.shape[0], _ptr(cache["k_cache"]), _ptr(cache["v_cache"]),
            _ptr(cache["k_scale"]), _ptr(cache["v_scale"]))
        if rc:
            raise ValueError(f"orc_kv_quantize_write_rope rejected its arguments ({rc})")
        return q_int8, q_scale

    def round_bf16(self, x):
        """fp32 -> nearest bf16 (ties to even), as fp32 values."""
        x = _c(x, np.float32)
        y = np.empty_like(x)
        self.lib.orc_round_bf16(_ptr(x), x.size, _ptr(y))
        return y

    def rope_rotate(self, x, positions, cos_sin):
        """The rotation alone: x [n, D] fp32 (a rotated copy is returned)."""
        x = _c(x, np.float32).copy()
        pos = _c(positions, np.int32)
        cs = _c(cos_sin, np.float32)
        rc = self.lib.orc_rope_rotate(x.shape[0], x.shape[1], _ptr(x), _ptr(pos), _ptr(cs),
                                      cs.shape[1], cs.shape[0])
        if rc:
            raise ValueError(f"orc_rope_rotate rejected its arguments ({rc})")
        return x

    def fill(self, wl):
        """Write every cache token of a workload; quantize its query tokens.

        History tokens go first (no query), then the query tokens in order.
        Returns ``(cache, q_int8 [Tq,Hq,D], q_scale [Tq,Hq])``.
        """
        cache = self.empty_cache(wl.num_blocks, wl.num_kv_heads, wl.head_dim, wl.block_size)
        is_q = np.zeros(wl.num_tokens, bool)
        is_q[wl.query_token_index] = True
        hist = np.nonzero(~is_q)[0]
        if hist.size:
            self.kv_quantize_write(wl.key[hist], wl.value[hist], wl.slot_mapping[hist],
                                   cache, num_q_heads=wl.num_q_heads)
        qi = wl.query_token_index
        q_int8, q_scale = self.kv_quantize_write(
            wl.key[qi], wl.value[qi], wl.slot_mapping[qi], cache,
            num_q_heads=wl.num_q_heads, query=wl.query)
        return cache, q_int8, q_scale

    # ------------------------------------------------------------------
    def paged_decode(self, q_int8, q_scale, cache, block_tables, seq_lens, *,
                     num_q_heads, w_group=32, partition=256, softmax_scale=None,
                     flags=0):
        q_int8 = _c(q_int8, np.int8)
        q_scale = _c(q_scale, np.float32)
        bt = _c(block_tables, np.int32)
        sl = _c(seq_lens, np.int32)
        nb, Hkv, _, bs, _ = cache["k_cache"].shape
        S, Hq, D = q_int8.shape
        assert Hq == num_q_heads
        if softmax_scale is None:
            softmax_scale = float(np.float32(1.0 / np.sqrt(D)))
        out = np.zeros((S, Hq, D), np.float32)
        rc = self.lib.orc_paged_decode(
            Hq, Hkv, D, bs, nb, S, _ptr(q_int8), _ptr(q_scale), _ptr(cache["k_cache"]),
            _ptr(cache["v_cache"]), _ptr(cache["k_scale"]), _ptr(cache["v_scale"]),
            _ptr(bt), bt.shape[1], _ptr(sl), partition, w_group, softmax_scale, flags,
            _ptr(out))
        if rc:
            raise ValueError(f"orc_paged_decode rejected its arguments ({rc})")
        return out

    def paged_decode_bf16qk(self, q_bf16, cache, block_tables, seq_lens, *, w_group=32,
                            partition=256, softmax_scale=None, flags=0):
        """BF16-QK ablation: the bf16 query (uint16 bits [S, Hq, D], not
        quantized) against the int8 K codes; the rest as paged_decode."""
        q = _c(q_bf16, np.uint16)
        bt = _c(block_tables, np.int32)
        sl = _c(seq_lens, np.int32)
        nb, Hkv, _, bs, _ = cache["k_cache"].shape
        S, Hq, D = q.shape
        if softmax_scale is None:
            softmax_scale = float(np.float32(1.0 / np.sqrt(D)))
        out = np.zeros((S, Hq, D), np.float32)
        rc = self.lib.orc_paged_decode_bf16qk(
            Hq, Hkv, D, bs, nb, S, _ptr(q), _ptr(cache["k_cache"]), _ptr(cache["v_cache"]),
            _ptr(cache["k_scale"]), _ptr(cache["v_scale"]), _ptr(bt), bt.shape[1], _ptr(sl),
            partition, w_group, softmax_scale, flags, _ptr(out))
        if rc:
            raise ValueError(f"orc_paged_decode_bf16qk rejected its arguments ({rc})")
        return out

    def paged_decode_multi(self, q_int8, q_scale, cache, block_tables, seq_lens, *,
                           num_q_heads, queries_per_seq, w_group=32, partition=256,
                           softmax_scale=None, flags=0):
        """Several causal queries per sequence (rows s * nq + j, query j at
        position L - nq + j): each is the one-query decode of the sequence cut
        after its own position -- orc_paged_decode over nq "sequences" per
        sequence, sharing its block table.  No arithmetic of its own."""
        nq = int(queries_per_seq)
        sl = _c(seq_lens, np.int32).astype(np.int64)
        S = sl.shape[0]
        cut = np.maximum(sl[:, None] - nq + np.arange(nq)[None, :] + 1, 0).reshape(-1)
        bt = np.repeat(_c(block_tables, np.int32), nq, axis=0)
        return self.paged_decode(q_int8, q_scale, cache, bt, cut.astype(np.int32),
                                 num_q_heads=num_q_heads, w_group=w_group, partition=partition,
                                 softmax_scale=softmax_scale, flags=flags)

    def decode_head(self, q_int8, q_scale, cache, block_tables, seq_lens, seq, head, *,
                    w_group=32, partition=256, softmax_scale=None, flags=0):
        """One (seq, q head) with every intermediate; returns a dict."""
        q_int8 = _c(q_int8, np.int8)
        q_scale = _c(q_scale, np.float32)
        bt = _c(block_tables, np.int32)
        sl = _c(seq_lens, np.int32)
        nb, Hkv, _, bs, _ = cache["k_cache"].shape
        S, Hq, D = q_int8.shape
        if softmax_scale is None:
            softmax_scale = float(np.float32(1.0 / np.sqrt(D)))
        L = int(sl[seq])
        NP = max(1, -(-L // partition))
        NG = max(1, -(-L // w_group))
        t = dict(s=np.zeros(L, np.float32), P=np.zeros(L, np.float32),
                 W=np.zeros(L, np.float32), Wq=np.zeros(L, np.int8),
                 sW=np.zeros(NG, np.float32), m=np.zeros(NP, np.float32),
                 l=np.zeros(NP, np.float32), o=np.zeros((NP, D), np.float64),
                 acc=np.zeros(L, np.int32))
        tr = _DecodeTrace(**{k: v.ctypes.data for k, v in t.items()})
        out = np.zeros(D, np.float32)
        rc = self.lib.orc_decode_head(
            Hq, Hkv, D, bs, nb, seq, head, _ptr(q_int8), _ptr(q_scale),
            _ptr(cache["k_cache"]), _ptr(cache["v_cache"]), _ptr(cache["k_scale"]),
            _ptr(cache["v_scale"]), _ptr(bt), bt.shape[1], _ptr(sl), partition, w_group,
            softmax_scale, flags, C.byref(tr), _ptr(out))
        if rc:
            raise ValueError(f"orc_decode_head rejected its arguments ({rc})")
        t["out"] = out
        return t

    # ------------------------------------------------------------------
    def prefix_prefill(self, q_int8, q_scale, query_start_loc, seq_lens, cache,
                       block_tables, *, w_group=32, tile=256, softmax_scale=None,
                       flags=0, rows=None, out=None):
        q_int8 = _c(q_int8, np.int8)
        q_scale = _c(q_scale, np.float32)
        qsl = _c(query_start_loc, np.int32)
        sl = _c(seq_lens, np.int32)
        bt = _c(block_tables, np.int32)
        nb, Hkv, _, bs, _ = cache["k_cache"].shape
        Tq, Hq, D = q_int8.shape
        if softmax_scale is None:
            softmax_scale = float(np.float32(1.0 / np.sqrt(D)))
        if out is None:
            out = np.zeros((Tq, Hq, D), np.float32)
        r = None if rows is None else _c(rows, np.int32)
        rc = self.lib.orc_prefix_prefill(
            Hq, Hkv, D, bs, nb, sl.shape[0], Tq, _ptr(q_int8), _ptr(q_scale), _ptr(qsl),
            _ptr(sl), _ptr(cache["k_cache"]), _ptr(cache["v_cache"]), _ptr(cache["k_scale"]),
            _ptr(cache["v_scale"]), _ptr(bt), bt.shape[1], tile, w_group, softmax_scale,
            flags, _ptr(r), 0 if r is None else r.shape[0], _ptr(out))
        if rc:
            raise ValueError(f"orc_prefix_prefill rejected its arguments ({rc})")
        return out

    def prefix_prefill_bf16qk(self, q_bf16, query_start_loc, seq_lens, cache, block_tables,
                              *, w_group=32, tile=256, softmax_scale=None, flags=0, rows=None,
                              out=None):
        """BF16-QK ablation of prefix_prefill: q_bf16 uint16 bits [Tq, Hq, D]."""
        q = _c(q_bf16, np.uint16)
        qsl = _c(query_start_loc, np.int32)
        sl = _c(seq_lens, np.int32)
        bt = _c(block_tables, np.int32)
        nb, Hkv, _, bs, _ = cache["k_cache"].shape
        Tq, Hq, D = q.shape
        if softmax_scale is None:
            softmax_scale = float(np.float32(1.0 / np.sqrt(D)))
        if out is None:
            out = np.zeros((Tq, Hq, D), np.float32)
        r = None if rows is None else _c(rows, np.int32)
        rc = self.lib.orc_prefix_prefill_bf16qk(
            Hq, Hkv, D, bs, nb, sl.shape[0], Tq, _ptr(q), _ptr(qsl), _ptr(sl),
            _ptr(cache["k_cache"]), _ptr(cache["v_cache"]), _ptr(cache["k_scale"]),
            _ptr(cache["v_scale"]), _ptr(bt), bt.shape[1], tile, w_group, softmax_scale, flags,
            _ptr(r), 0 if r is None else r.shape[0], _ptr(out))
        if rc:
            raise ValueError(f"orc_prefix_prefill_bf16qk rejected its arguments ({rc})")
        return out

    def prefill_row(self, q_int8, q_scale, query_start_loc, seq_lens, cache,
                    block_tables, row, head, *, w_group=32, tile=256,
                    softmax_scale=None, flags=0):
        q_int8 = _c(q_int8, np.int8)
        q_scale = _c(q_scale, np.float32)
        qsl = _c(query_start_loc, np.int32)
        sl = _c(seq_lens, np.int32)
        bt = _c(block_tables, np.int32)
        nb, Hkv, _, bs, _ = cache["k_cache"].shape
        Tq, Hq, D = q_int8.shape
        if softmax_scale is None:
            softmax_scale = float(np.float32(1.0 / np.sqrt(D)))
        b = int(np.searchsorted(qsl, row, side="right") - 1)
        chunk = int(qsl[b + 1] - qsl[b])
        nk = int(sl[b]) - chunk + (row - int(qsl[b])) + 1
        # Buffers cover the whole sequence, so a row can never write past them.
        cap = max(int(sl[b]), nk)
        t = dict(s=np.zeros(cap, np.float32), ptil=np.zeros(cap, np.float32),
                 Wq=np.zeros(cap, np.int8), sW=np.zeros(-(-cap // w_group), np.float32),
                 m_tile=np.zeros(-(-cap // tile), np.float32), l=np.zeros(1, np.float64))
        tr = _PrefillTrace(**{k: v.ctypes.data for k, v in t.items()})
        out = np.zeros(D, np.float32)
        rc = self.lib.orc_prefill_row(
            Hq, Hkv, D, bs, nb, sl.shape[0], Tq, row, head, _ptr(q_int8), _ptr(q_scale),
            _ptr(qsl), _ptr(sl), _ptr(cache["k_cache"]), _ptr(cache["v_cache"]),
            _ptr(cache["k_scale"]), _ptr(cache["v_scale"]), _ptr(bt), bt.shape[1], tile,
            w_group, softmax_scale, flags, C.byref(tr), _ptr(out))
        if rc:
            raise ValueError(f"orc_prefill_row rejected its arguments ({rc})")
        for k, n in (("s", nk), ("ptil", nk), ("Wq", nk), ("sW", -(-nk // w_group)),
                     ("m_tile", -(-nk // tile))):
            t[k] = t[k][:n]
        t["out"] = out
        t["nk"] = nk
        return t


_default: Optional[Oracle] = None


def default() -> Oracle:
    """The oracle built from ``oracle.cpp`` (built on first use)."""
    global _default
    if _default is None:
        _default = Oracle()
    return _default
