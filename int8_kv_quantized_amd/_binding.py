"""ctypes binding of libi8kv.so: argument marshalling and host-side shape checks.

Names follow the C ABI in include/i8kv.h without the ``i8kv_`` prefix.
Tensor arguments may be torch tensors on the GPU (checked for dtype, shape,
contiguity and device) or raw device pointers (ints, trusted as given).
"""
from __future__ import annotations

import contextlib
import ctypes as C
import dataclasses
import functools
import math
from pathlib import Path
from typing import Optional

HERE = Path(__file__).resolve().parent
I8KV_OK = 0
_STATUS = {0: "ok", 1: "null pointer argument", 2: "invalid argument",
           3: "unsupported shape or parameter", 4: "workspace missing or too small",
           5: "kernel launch failed"}


class I8KVError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: status {status} ({_STATUS.get(status, 'unknown')})")
        self.status = status


PV_VARIANTS = {"int8": 0, "bf16": 1, "uint8": 2}


class DecodeOpts(C.Structure):
    _fields_ = [("partition_size", C.c_int32), ("w_group", C.c_int32),
                ("softmax_scale", C.c_float), ("pv", C.c_int32),
                ("queries_per_seq", C.c_int32), ("out_bf16", C.c_int32)]


class PrefillOpts(C.Structure):
    _fields_ = [("w_group", C.c_int32), ("softmax_scale", C.c_float), ("pv", C.c_int32),
                ("out_bf16", C.c_int32)]


class CacheDesc(C.Structure):
    _fields_ = [("num_q_heads", C.c_int32), ("num_kv_heads", C.c_int32),
                ("head_dim", C.c_int32), ("block_size", C.c_int32),
                ("num_blocks", C.c_int32)]

    def __init__(self, num_q_heads, num_kv_heads, head_dim, num_blocks, block_size=16):
        super().__init__(num_q_heads, num_kv_heads, head_dim, block_size, num_blocks)

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    def __repr__(self):
        return (f"CacheDesc(Hq={self.num_q_heads}, Hkv={self.num_kv_heads}, "
                f"D={self.head_dim}, bs={self.block_size}, nb={self.num_blocks})")


_lib = None


def lib_path() -> Path:
    return HERE / "libi8kv.so"


def load_library():
    """Load libi8kv.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    p = lib_path()
    if not p.exists():
        raise RuntimeError(f"{p} is missing: build it with int8_kv_quantized_amd.build.build() "
                           "(there is no fallback path)")
    # torch first: it brings its own HIP runtime into the process, and the
    # library must bind to that same runtime.  Loaded before torch, the library
    # pulls in the system one, torch then shares a runtime it was not built
    # with, and launches fail with hipErrorNoDevice.
    import torch  # noqa: F401
    lib = C.CDLL(str(p))
    P, I32, F, SZ = C.c_void_p, C.c_int32, C.c_float, C.c_size_t
    D = C.POINTER(CacheDesc)
    lib.i8kv_abi_version.restype = I32
    lib.i8kv_abi_version.argtypes = []
    lib.i8kv_status_string.restype = C.c_char_p
    lib.i8kv_status_string.argtypes = [C.c_int32]
    lib.i8kv_kv_quantize_write.restype = C.c_int
    lib.i8kv_kv_quantize_write.argtypes = [D, I32] + [P] * 10 + [P]
    lib.i8kv_kv_quantize_write_rope.restype = C.c_int
    lib.i8kv_kv_quantize_write_rope.argtypes = [D, I32] + [P] * 8 + [I32, I32] + [P] * 4 + [P]
    lib.i8kv_paged_decode_workspace_bytes.restype = SZ
    lib.i8kv_paged_decode_workspace_bytes.argtypes = [D, I32, I32, I32]
    lib.i8kv_paged_decode_int8.restype = C.c_int
    lib.i8kv_paged_decode_int8.argtypes = ([D, I32] + [P] * 7 + [I32, P, I32, I32, I32, F, P, SZ,
                                                                 P, P])
    lib.i8kv_paged_decode_noalloc_max_bytes.restype = SZ
    lib.i8kv_paged_decode_noalloc_max_bytes.argtypes = []
    lib.i8kv_paged_decode_int8_noalloc.restype = C.c_int
    lib.i8kv_paged_decode_int8_noalloc.argtypes = ([D, I32] + [P] * 7 + [I32, P, I32, I32, I32, F,
                                                                         P, P])
    lib.i8kv_paged_decode_partials.restype = C.c_int
    lib.i8kv_paged_decode_partials.argtypes = ([D, I32] + [P] * 7 + [I32, P, I32, I32, I32, F, P,
                                                                     SZ, P])
    lib.i8kv_paged_decode_merge.restype = C.c_int
    lib.i8kv_paged_decode_merge.argtypes = [D, I32, P, I32, I32, P, SZ, P, P]
    lib.i8kv_paged_decode_uint8w.restype = C.c_int
    lib.i8kv_paged_decode_uint8w.argtypes = ([D, I32] + [P] * 7 + [I32, P, I32, I32, I32, F, P, SZ, P, P])
    O = C.POINTER(DecodeOpts)
    lib.i8kv_paged_decode_ex_workspace_bytes.restype = SZ
    lib.i8kv_paged_decode_ex_workspace_bytes.argtypes = [D, O, I32, I32]
    lib.i8kv_paged_decode_ex.restype = C.c_int
    lib.i8kv_paged_decode_ex.argtypes = ([D, O, I32] + [P] * 7 + [I32, P, I32, P, SZ, P, P])
    lib.i8kv_paged_decode_bf16pv.restype = C.c_int
    lib.i8kv_paged_decode_bf16pv.argtypes = ([D, I32] + [P] * 7 + [I32, P, I32, I32, F, P, SZ, P, P])
    lib.i8kv_paged_decode_bf16qk.restype = C.c_int
    lib.i8kv_paged_decode_bf16qk.argtypes = ([D, I32] + [P] * 6 + [I32, P, I32, I32, I32, F, P, SZ,
                                                                  P, P])
    lib.i8kv_decode_step_int8.restype = C.c_int
    lib.i8kv_decode_step_int8.argtypes = ([D, I32] + [P] * 10 + [I32, P, I32, I32, I32, F, P, SZ,
                                                                  P, P])
    lib.i8kv_prefix_prefill_workspace_bytes.restype = SZ
    lib.i8kv_prefix_prefill_workspace_bytes.argtypes = [D, I32, I32]
    lib.i8kv_prefix_prefill_bf16pv.restype = C.c_int
    lib.i8kv_prefix_prefill_bf16pv.argtypes = ([D, I32, I32, I32] + [P] * 9 + [I32, F, P, SZ, P, P])
    lib.i8kv_prefix_prefill_bf16qk.restype = C.c_int
    lib.i8kv_prefix_prefill_bf16qk.argtypes = ([D, I32, I32, I32] + [P] * 8 + [I32, I32, F, P,
                                                                              SZ, P, P])
    lib.i8kv_prefix_prefill_uint8w.restype = C.c_int
    lib.i8kv_prefix_prefill_uint8w.argtypes = ([D, I32, I32, I32] + [P] * 9 + [I32, I32, F, P, SZ,
                                                                              P, P])
    lib.i8kv_prefix_prefill_ex.restype = C.c_int
    lib.i8kv_prefix_prefill_ex.argtypes = ([D, C.POINTER(PrefillOpts), I32, I32, I32] + [P] * 9
                                           + [I32, P, P])
    lib.i8kv_prefix_prefill_int8.restype = C.c_int
    lib.i8kv_prefix_prefill_int8.argtypes = ([D, I32, I32, I32] + [P] * 9 + [I32, I32, F, P, SZ,
                                                                            P, P])
    _lib = lib
    return lib


def abi_version() -> int:
    return int(load_library().i8kv_abi_version())


def status_string(status: int) -> str:
    return load_library().i8kv_status_string(int(status)).decode()


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------
def _is_tensor(x) -> bool:
    return hasattr(x, "data_ptr") and hasattr(x, "dtype")


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return C.c_void_p(x)
    if _is_tensor(x):
        return C.c_void_p(x.data_ptr())
    raise TypeError(f"expected a tensor, a device pointer or None, got {type(x)}")


def _check(x, name, dtype, shape=None):
    """Validate a torch tensor argument (raw pointers are passed through)."""
    if x is None or isinstance(x, int):
        return
    import torch
    ok = x.dtype in dtype if isinstance(dtype, tuple) else x.dtype == dtype
    if not ok:
        raise ValueError(f"{name}: dtype {x.dtype}, expected {dtype}")
    if not x.is_cuda:
        raise ValueError(f"{name}: must be a GPU tensor")
    if not x.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if shape is not None:
        want = tuple(int(s) for s in shape)
        if tuple(x.shape) != want:
            raise ValueError(f"{name}: shape {tuple(x.shape)}, expected {want}")
    del torch


def _stream(stream):
    if stream is None:
        import torch
        return C.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return C.c_void_p(stream)
    return C.c_void_p(stream.cuda_stream)


def _on_stream(stream):
    """Context that makes ``stream`` torch's current stream (None: leave it)."""
    if stream is None:
        return contextlib.nullcontext()
    import torch
    if isinstance(stream, int):
        if stream == torch.cuda.current_stream().cuda_stream:
            return contextlib.nullcontext()
        stream = torch.cuda.ExternalStream(stream)
    return torch.cuda.stream(stream)


def _allocates_on_stream(fn):
    """Run an entry point with its ``stream`` keyword as torch's current stream.

    Every tensor the binding allocates for the call (workspace, outputs, the
    quantized queries) is then allocated -- and zero-filled -- on the stream
    the kernels are enqueued on: the fill is ordered before the launch, and
    torch's caching allocator hands the block to a later allocation only
    after the work queued on that stream, never while the kernels may still
    use it.  ``stream`` must be passed by keyword.
    """
    @functools.wraps(fn)
    def wrapper(*args, stream=None, **kw):
        with _on_stream(stream):
            return fn(*args, stream=stream, **kw)
    return wrapper


def _raise(fn, st):
    if st != I8KV_OK:
        raise I8KVError(fn, st)


@dataclasses.dataclass
class PagedCache:
    """Device tensors of one paged int8 cache (layouts of include/i8kv.h)."""
    k_cache: object   # int8  [nb, Hkv, D/16, 16, 16]
    v_cache: object   # int8  [nb, Hkv, D, 16]
    k_scale: object   # fp32  [nb, 16, Hkv]
    v_scale: object   # fp32  [nb, 16, Hkv]

    @classmethod
    def allocate(cls, desc: CacheDesc, device="cuda", zero=True):
        import torch
        nb, H, D, bs = desc.num_blocks, desc.num_kv_heads, desc.head_dim, desc.block_size
        mk = torch.zeros if zero else torch.empty
        return cls(mk((nb, H, D // 16, bs, 16), dtype=torch.int8, device=device),
                   mk((nb, H, D, bs), dtype=torch.int8, device=device),
                   mk((nb, bs, H), dtype=torch.float32, device=device),
                   mk((nb, bs, H), dtype=torch.float32, device=device))

    def check(self, desc: CacheDesc):
        import torch
        nb, H, D, bs = desc.num_blocks, desc.num_kv_heads, desc.head_dim, desc.block_size
        _check(self.k_cache, "k_cache", torch.int8, (nb, H, D // 16, bs, 16))
        _check(self.v_cache, "v_cache", torch.int8, (nb, H, D, bs))
        _check(self.k_scale, "k_scale", torch.float32, (nb, bs, H))
        _check(self.v_scale, "v_scale", torch.float32, (nb, bs, H))


# ---------------------------------------------------------------------------
# the three operations
# ---------------------------------------------------------------------------
def _producer_args(desc: CacheDesc, key, value, slot_mapping, cache: PagedCache, query,
                   q_int8, q_scale, num_tokens):
    import torch
    if num_tokens is None:
        num_tokens = int(key.shape[0])
    T, Hq, Hkv, D = num_tokens, desc.num_q_heads, desc.num_kv_heads, desc.head_dim
    bits16 = (torch.bfloat16, torch.int16, torch.uint16)
    _check(key, "key", bits16)
    _check(value, "value", bits16)
    _check(query, "query", bits16)
    for name, x in (("key", key), ("value", value)):
        if _is_tensor(x) and tuple(x.shape) != (T, Hkv, D):
            raise ValueError(f"{name}: shape {tuple(x.shape)}, expected {(T, Hkv, D)}")
    _check(slot_mapping, "slot_mapping", torch.int32, (T,))
    cache.check(desc)
    if query is not None:
        if _is_tensor(query) and tuple(query.shape) != (T, Hq, D):
            raise ValueError(f"query: shape {tuple(query.shape)}, expected {(T, Hq, D)}")
        if q_int8 is None:
            q_int8 = torch.empty((T, Hq, D), dtype=torch.int8, device=key.device)
        if q_scale is None:
            q_scale = torch.empty((T, Hq), dtype=torch.float32, device=key.device)
        _check(q_int8, "q_int8", torch.int8, (T, Hq, D))
        _check(q_scale, "q_scale", torch.float32, (T, Hq))
    return T, q_int8, q_scale


@_allocates_on_stream
def kv_quantize_write(desc: CacheDesc, key, value, slot_mapping, cache: PagedCache,
                      query=None, q_int8=None, q_scale=None, num_tokens: Optional[int] = None,
                      stream=None):
    """Fused producer: quantize K/V (and Q) and write the paged cache.

    Returns ``(q_int8, q_scale)`` (allocated here when ``query`` is given and
    they are not).
    """
    lib = load_library()
    T, q_int8, q_scale = _producer_args(desc, key, value, slot_mapping, cache, query, q_int8,
                                        q_scale, num_tokens)
    st = lib.i8kv_kv_quantize_write(
        C.byref(desc), T, _ptr(key), _ptr(value), _ptr(query), _ptr(q_int8), _ptr(q_scale),
        _ptr(slot_mapping), _ptr(cache.k_cache), _ptr(cache.v_cache), _ptr(cache.k_scale),
        _ptr(cache.v_scale), _stream(stream))
    _raise("kv_quantize_write", st)
    return q_int8, q_scale


@_allocates_on_stream
def kv_quantize_write_rope(desc: CacheDesc, key, value, slot_mapping, positions, cos_sin,
                           cache: PagedCache, query=None, q_int8=None, q_scale=None,
                           num_tokens: Optional[int] = None, rotary_dim: Optional[int] = None,
                           max_position: Optional[int] = None, stream=None):
    """The producer with the rotary embedding of Q and K fused in.

    ``positions`` [T] int32; ``cos_sin`` [max_position, rotary_dim] fp32
    (cosines, then sines).  Returns ``(q_int8, q_scale)`` as kv_quantize_write.
    """
    import torch
    lib = load_library()
    T, q_int8, q_scale = _producer_args(desc, key, value, slot_mapping, cache, query, q_int8,
                                        q_scale, num_tokens)
    _check(positions, "positions", torch.int32, (T,))
    _check(cos_sin, "cos_sin", torch.float32)
    if _is_tensor(cos_sin):
        if cos_sin.dim() != 2:
            raise ValueError(f"cos_sin: shape {tuple(cos_sin.shape)}, expected (P, R)")
        max_position = int(cos_sin.shape[0]) if max_position is None else max_position
        rotary_dim = int(cos_sin.shape[1]) if rotary_dim is None else rotary_dim
    if rotary_dim is None or max_position is None:
        raise ValueError("rotary_dim and max_position are needed with a raw cos_sin pointer")
    st = lib.i8kv_kv_quantize_write_rope(
        C.byref(desc), T, _ptr(key), _ptr(value), _ptr(query), _ptr(q_int8), _ptr(q_scale),
        _ptr(slot_mapping), _ptr(positions), _ptr(cos_sin), int(rotary_dim), int(max_position),
        _ptr(cache.k_cache), _ptr(cache.v_cache), _ptr(cache.k_scale), _ptr(cache.v_scale),
        _stream(stream))
    _raise("kv_quantize_write_rope", st)
    return q_int8, q_scale


def paged_decode_workspace_bytes(desc: CacheDesc, num_seqs: int, max_seq_len: int,
                                 partition_size: int = 256) -> int:
    return int(load_library().i8kv_paged_decode_workspace_bytes(
        C.byref(desc), int(num_seqs), int(max_seq_len), int(partition_size)))


def _decode_args(desc: CacheDesc, q_int8, q_scale, cache: PagedCache, block_tables, seq_lens,
                 max_seq_len, partition_size, softmax_scale, workspace, out, q_bf16=None,
                 want_out=True):
    import torch
    q_any = q_int8 if q_bf16 is None else q_bf16
    S = int(seq_lens.shape[0]) if _is_tensor(seq_lens) else int(q_any.shape[0])
    Hq, D = desc.num_q_heads, desc.head_dim
    if q_bf16 is None:
        _check(q_int8, "q_int8", torch.int8, (S, Hq, D))
        _check(q_scale, "q_scale", torch.float32, (S, Hq))
    else:
        _check(q_bf16, "query", (torch.bfloat16, torch.int16, torch.uint16), (S, Hq, D))
    cache.check(desc)
    _check(block_tables, "block_tables", torch.int32)
    if not _is_tensor(block_tables):
        raise ValueError("block_tables must be a tensor (its width is needed)")
    if block_tables.dim() != 2 or block_tables.shape[0] != S:
        raise ValueError(f"block_tables: shape {tuple(block_tables.shape)}, expected ({S}, *)")
    _check(seq_lens, "seq_lens", torch.int32, (S,))
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    need = paged_decode_workspace_bytes(desc, S, max_seq_len, partition_size)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=block_tables.device)
    ws_bytes = workspace.numel() * workspace.element_size() if _is_tensor(workspace) else need
    if want_out:
        if out is None:
            out = torch.empty((S, Hq, D), dtype=torch.float32, device=block_tables.device)
        _check(out, "out", torch.float32, (S, Hq, D))
    return S, float(softmax_scale), workspace, int(ws_bytes), out


@_allocates_on_stream
def paged_decode_int8(desc: CacheDesc, q_int8, q_scale, cache: PagedCache, block_tables,
                      seq_lens, max_seq_len: int, w_group: int = 32,
                      partition_size: int = 256, softmax_scale: Optional[float] = None,
                      workspace=None, out=None, stream=None):
    """Paged decode over the int8 cache; returns ``out`` [S, Hq, D] fp32.

    ``workspace`` must hold paged_decode_workspace_bytes(...) bytes and be
    256-byte aligned (allocated here if None); its contents need no
    initialization.
    """
    lib = load_library()
    S, scale, workspace, ws_bytes, out = _decode_args(
        desc, q_int8, q_scale, cache, block_tables, seq_lens, max_seq_len, partition_size,
        softmax_scale, workspace, out)
    st = lib.i8kv_paged_decode_int8(
        C.byref(desc), S, _ptr(q_int8), _ptr(q_scale), _ptr(cache.k_cache),
        _ptr(cache.v_cache), _ptr(cache.k_scale), _ptr(cache.v_scale), _ptr(block_tables),
        int(block_tables.shape[1]), _ptr(seq_lens), int(max_seq_len), int(partition_size),
        int(w_group), scale, _ptr(workspace), ws_bytes, _ptr(out), _stream(stream))
    _raise("paged_decode_int8", st)
    return out


def paged_decode_noalloc_max_bytes() -> int:
    return int(load_library().i8kv_paged_decode_noalloc_max_bytes())


@_allocates_on_stream
def paged_decode_int8_noalloc(desc: CacheDesc, q_int8, q_scale, cache: PagedCache,
                              block_tables, seq_lens, max_seq_len: int, w_group: int = 32,
                              partition_size: int = 256, softmax_scale: Optional[float] = None,
                              out=None, stream=None):
    """paged_decode_int8 without a workspace: the library's fixed per-GPU
    array holds the partials (see include/i8kv.h for the size limit; calls
    that overlap on one GPU race).  With ``out`` given, nothing is allocated."""
    lib = load_library()
    S, scale, _, _, out = _decode_args(
        desc, q_int8, q_scale, cache, block_tables, seq_lens, max_seq_len, partition_size,
        softmax_scale, 0, out)
    st = lib.i8kv_paged_decode_int8_noalloc(
        C.byref(desc), S, _ptr(q_int8), _ptr(q_scale), _ptr(cache.k_cache),
        _ptr(cache.v_cache), _ptr(cache.k_scale), _ptr(cache.v_scale), _ptr(block_tables),
        int(block_tables.shape[1]), _ptr(seq_lens), int(max_seq_len), int(partition_size),
        int(w_group), scale, _ptr(out), _stream(stream))
    _raise("paged_decode_int8_noalloc", st)
    return out


@_allocates_on_stream
def paged_decode_partials(desc: CacheDesc, q_int8, q_scale, cache: PagedCache, block_tables,
                          seq_lens, max_seq_len: int, w_group: int = 32,
                          partition_size: int = 256, softmax_scale: Optional[float] = None,
                          workspace=None, stream=None):
    """Stage 1 of paged_decode_int8 alone: every sequence's per-partition
    (m_p, l_p, o_p) into ``workspace`` (layout in include/i8kv.h); returns
    the workspace (allocated here if None)."""
    lib = load_library()
    S, scale, workspace, ws_bytes, _ = _decode_args(
        desc, q_int8, q_scale, cache, block_tables, seq_lens, max_seq_len, partition_size,
        softmax_scale, workspace, None, want_out=False)
    st = lib.i8kv_paged_decode_partials(
        C.byref(desc), S, _ptr(q_int8), _ptr(q_scale), _ptr(cache.k_cache),
        _ptr(cache.v_cache), _ptr(cache.k_scale), _ptr(cache.v_scale), _ptr(block_tables),
        int(block_tables.shape[1]), _ptr(seq_lens), int(max_seq_len), int(partition_size),
        int(w_group), scale, _ptr(workspace), ws_bytes, _stream(stream))
    _raise("paged_decode_partials", st)
    return workspace


@_allocates_on_stream
def paged_decode_merge(desc: CacheDesc, seq_lens, max_seq_len: int, workspace,
                       partition_size: int = 256, out=None, stream=None):
    """Stage 2 of paged_decode_int8 alone: merge the partials in ``workspace``
    into ``out`` [S, Hq, D] fp32 (allocated here if None)."""
    import torch
    lib = load_library()
    _check(seq_lens, "seq_lens", torch.int32)
    S = int(seq_lens.shape[0])
    Hq, D = desc.num_q_heads, desc.head_dim
    if workspace is None:
        raise ValueError("workspace: the partials to merge are needed")
    need = paged_decode_workspace_bytes(desc, S, max_seq_len, partition_size)
    ws_bytes = workspace.numel() * workspace.element_size() if _is_tensor(workspace) else need
    if out is None:
        out = torch.empty((S, Hq, D), dtype=torch.float32, device=seq_lens.device)
    _check(out, "out", torch.float32, (S, Hq, D))
    st = lib.i8kv_paged_decode_merge(C.byref(desc), S, _ptr(seq_lens), int(max_seq_len),
                                     int(partition_size), _ptr(workspace), int(ws_bytes),
                                     _ptr(out), _stream(stream))
    _raise("paged_decode_merge", st)
    return out


@_allocates_on_stream
def paged_decode_uint8w(desc: CacheDesc, q_int8, q_scale, cache: PagedCache, block_tables,
                        seq_lens, max_seq_len: int, w_group: int = 32,
                        partition_size: int = 256, softmax_scale: Optional[float] = None,
                        workspace=None, out=None, stream=None):
    """The decode with UINT8 W groups (sW = max W / 255, codes 0..255); same
    arguments as paged_decode_int8."""
    lib = load_library()
    S, scale, workspace, ws_bytes, out = _decode_args(
        desc, q_int8, q_scale, cache, block_tables, seq_lens, max_seq_len, partition_size,
        softmax_scale, workspace, out)
    st = lib.i8kv_paged_decode_uint8w(
        C.byref(desc), S, _ptr(q_int8), _ptr(q_scale), _ptr(cache.k_cache),
        _ptr(cache.v_cache), _ptr(cache.k_scale), _ptr(cache.v_scale), _ptr(block_tables),
        int(block_tables.shape[1]), _ptr(seq_lens), int(max_seq_len), int(partition_size),
        int(w_group), scale, _ptr(workspace), ws_bytes, _ptr(out), _stream(stream))
    _raise("paged_decode_uint8w", st)
    return out


def paged_decode_ex_workspace_bytes(desc: CacheDesc, opts: DecodeOpts, num_seqs: int,
                                    max_seq_len: int) -> int:
    return int(load_library().i8kv_paged_decode_ex_workspace_bytes(
        C.byref(desc), C.byref(opts), int(num_seqs), int(max_seq_len)))


@_allocates_on_stream
def paged_decode_ex(desc: CacheDesc, q_int8, q_scale, cache: PagedCache, block_tables, seq_lens,
                    max_seq_len: int, queries_per_seq: int = 1, pv: str = "int8",
                    w_group: int = 32, out_bf16: bool = False, partition_size: int = 256,
                    softmax_scale: Optional[float] = None, workspace=None, out=None,
                    stream=None):
    """The decode with options: nq causal queries per sequence (rows
    s * nq + j of q_int8 / q_scale / out), the PV variant ("int8", "bf16",
    "uint8") and a bf16 output (returned as torch.bfloat16)."""
    import torch
    lib = load_library()
    nq = int(queries_per_seq)
    S = int(seq_lens.shape[0])
    Hq, D = desc.num_q_heads, desc.head_dim
    _check(q_int8, "q_int8", torch.int8, (S * nq, Hq, D))
    _check(q_scale, "q_scale", torch.float32, (S * nq, Hq))
    cache.check(desc)
    _check(block_tables, "block_tables", torch.int32)
    if not _is_tensor(block_tables) or block_tables.dim() != 2 or block_tables.shape[0] != S:
        raise ValueError(f"block_tables: expected a ({S}, *) int32 tensor")
    _check(seq_lens, "seq_lens", torch.int32, (S,))
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    if pv not in PV_VARIANTS:
        raise ValueError(f"pv must be one of {sorted(PV_VARIANTS)}")
    opts = DecodeOpts(int(partition_size), int(w_group), float(softmax_scale), PV_VARIANTS[pv],
                      nq, 1 if out_bf16 else 0)
    need = paged_decode_ex_workspace_bytes(desc, opts, S, max_seq_len)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=block_tables.device)
    ws_bytes = workspace.numel() * workspace.element_size() if _is_tensor(workspace) else need
    dt = torch.bfloat16 if out_bf16 else torch.float32
    if out is None:
        out = torch.empty((S * nq, Hq, D), dtype=dt, device=block_tables.device)
    _check(out, "out", dt, (S * nq, Hq, D))
    st = lib.i8kv_paged_decode_ex(
        C.byref(desc), C.byref(opts), S, _ptr(q_int8), _ptr(q_scale), _ptr(cache.k_cache),
        _ptr(cache.v_cache), _ptr(cache.k_scale), _ptr(cache.v_scale), _ptr(block_tables),
        int(block_tables.shape[1]), _ptr(seq_lens), int(max_seq_len), _ptr(workspace),
        int(ws_bytes), _ptr(out), _stream(stream))
    _raise("paged_decode_ex", st)
    return out


@_allocates_on_stream
def paged_decode_bf16pv(desc: CacheDesc, q_int8, q_scale, cache: PagedCache, block_tables,
                        seq_lens, max_seq_len: int, partition_size: int = 256,
                        softmax_scale: Optional[float] = None, workspace=None, out=None,
                        stream=None):
    """The BF16-PV ablation of paged_decode_int8 (W = P*sV in bf16 times the
    int8 V, no W groups); same arguments without w_group."""
    lib = load_library()
    S, scale, workspace, ws_bytes, out = _decode_args(
        desc, q_int8, q_scale, cache, block_tables, seq_lens, max_seq_len, partition_size,
        softmax_scale, workspace, out)
    st = lib.i8kv_paged_decode_bf16pv(
        C.byref(desc), S, _ptr(q_int8), _ptr(q_scale), _ptr(cache.k_cache),
        _ptr(cache.v_cache), _ptr(cache.k_scale), _ptr(cache.v_scale), _ptr(block_tables),
        int(block_tables.shape[1]), _ptr(seq_lens), int(max_seq_len), int(partition_size),
        scale, _ptr(workspace), ws_bytes, _ptr(out), _stream(stream))
    _raise("paged_decode_bf16pv", st)
    return out


@_allocates_on_stream
def paged_decode_bf16qk(desc: CacheDesc, query, cache: PagedCache, block_tables, seq_lens,
                        max_seq_len: int, w_group: int = 32, partition_size: int = 256,
                        softmax_scale: Optional[float] = None, workspace=None, out=None,
                        stream=None):
    """The BF16-QK ablation of paged_decode_int8: ``query`` [S, Hq, D] bf16
    (torch.bfloat16, or its bits as int16 / uint16), not quantized, against
    the int8 K codes; the other arguments as paged_decode_int8."""
    lib = load_library()
    S, scale, workspace, ws_bytes, out = _decode_args(
        desc, None, None, cache, block_tables, seq_lens, max_seq_len, partition_size,
        softmax_scale, workspace, out, q_bf16=query)
    st = lib.i8kv_paged_decode_bf16qk(
        C.byref(desc), S, _ptr(query), _ptr(cache.k_cache), _ptr(cache.v_cache),
        _ptr(cache.k_scale), _ptr(cache.v_scale), _ptr(block_tables),
        int(block_tables.shape[1]), _ptr(seq_lens), int(max_seq_len), int(partition_size),
        int(w_group), scale, _ptr(workspace), ws_bytes, _ptr(out), _stream(stream))
    _raise("paged_decode_bf16qk", st)
    return out


@_allocates_on_stream
def decode_step_int8(desc: CacheDesc, key, value, query, cache: PagedCache, block_tables,
                     seq_lens, max_seq_len: int, w_group: int = 32, partition_size: int = 256,
                     softmax_scale: Optional[float] = None, workspace=None, out=None,
                     q_int8=None, q_scale=None, stream=None):
    """One decode step with the producer fused in: writes each sequence's
    newest token (position seq_lens[s] - 1, bf16 ``key``/``value`` [S, Hkv, D])
    into ``cache`` and attends its ``query`` [S, Hq, D] over the sequence.
    Returns ``out`` [S, Hq, D] fp32; ``q_int8``/``q_scale`` are optional
    outputs (the quantized queries)."""
    import torch
    lib = load_library()
    S = int(seq_lens.shape[0]) if _is_tensor(seq_lens) else int(key.shape[0])
    Hq, Hkv, D = desc.num_q_heads, desc.num_kv_heads, desc.head_dim
    bits16 = (torch.bfloat16, torch.int16, torch.uint16)
    _check(key, "key", bits16, (S, Hkv, D))
    _check(value, "value", bits16, (S, Hkv, D))
    _check(query, "query", bits16, (S, Hq, D))
    if (q_int8 is None) != (q_scale is None):
        raise ValueError("q_int8 and q_scale go together")
    if q_int8 is not None:
        _check(q_int8, "q_int8", torch.int8, (S, Hq, D))
        _check(q_scale, "q_scale", torch.float32, (S, Hq))
    cache.check(desc)
    _check(block_tables, "block_tables", torch.int32)
    if not _is_tensor(block_tables):
        raise ValueError("block_tables must be a tensor (its width is needed)")
    if block_tables.dim() != 2 or block_tables.shape[0] != S:
        raise ValueError(f"block_tables: shape {tuple(block_tables.shape)}, expected ({S}, *)")
    _check(seq_lens, "seq_lens", torch.int32, (S,))
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    need = paged_decode_workspace_bytes(desc, S, max_seq_len, partition_size)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=block_tables.device)
    ws_bytes = workspace.numel() * workspace.element_size() if _is_tensor(workspace) else need
    if out is None:
        out = torch.empty((S, Hq, D), dtype=torch.float32, device=block_tables.device)
    _check(out, "out", torch.float32, (S, Hq, D))
    st = lib.i8kv_decode_step_int8(
        C.byref(desc), S, _ptr(key), _ptr(value), _ptr(query), _ptr(q_int8), _ptr(q_scale),
        _ptr(cache.k_cache), _ptr(cache.v_cache), _ptr(cache.k_scale), _ptr(cache.v_scale),
        _ptr(block_tables), int(block_tables.shape[1]), _ptr(seq_lens), int(max_seq_len),
        int(partition_size), int(w_group), float(softmax_scale), _ptr(workspace), int(ws_bytes),
        _ptr(out), _stream(stream))
    _raise("decode_step_int8", st)
    return out


def prefix_prefill_workspace_bytes(desc: CacheDesc, num_seqs: int, total_q: int) -> int:
    return int(load_library().i8kv_prefix_prefill_workspace_bytes(
        C.byref(desc), int(num_seqs), int(total_q)))


@_allocates_on_stream
def prefix_prefill_int8(desc: CacheDesc, q_int8, q_scale, query_start_loc, seq_lens,
                        cache: PagedCache, block_tables, max_query_len: int,
                        w_group: int = 32, softmax_scale: Optional[float] = None,
                        out=None, workspace=None, stream=None, _bf16pv=False, _uint8w=False):
    """Chunked prefill with history; returns ``out`` [total_q, Hq, D] fp32."""
    import torch
    lib = load_library()
    Tq = int(q_int8.shape[0])
    S = int(seq_lens.shape[0])
    Hq, D = desc.num_q_heads, desc.head_dim
    _check(q_int8, "q_int8", torch.int8, (Tq, Hq, D))
    _check(q_scale, "q_scale", torch.float32, (Tq, Hq))
    _check(query_start_loc, "query_start_loc", torch.int32, (S + 1,))
    _check(seq_lens, "seq_lens", torch.int32, (S,))
    cache.check(desc)
    _check(block_tables, "block_tables", torch.int32)
    if block_tables.dim() != 2 or block_tables.shape[0] != S:
        raise ValueError(f"block_tables: shape {tuple(block_tables.shape)}, expected ({S}, *)")
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((Tq, Hq, D), dtype=torch.float32, device=q_int8.device)
    _check(out, "out", torch.float32, (Tq, Hq, D))
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    common = (C.byref(desc), S, Tq, int(max_query_len), _ptr(q_int8), _ptr(q_scale),
              _ptr(query_start_loc), _ptr(seq_lens), _ptr(cache.k_cache), _ptr(cache.v_cache),
              _ptr(cache.k_scale), _ptr(cache.v_scale), _ptr(block_tables),
              int(block_tables.shape[1]))
    tail = (float(softmax_scale), _ptr(workspace), int(ws_bytes), _ptr(out), _stream(stream))
    if _bf16pv:
        st = lib.i8kv_prefix_prefill_bf16pv(*common, *tail)
        _raise("prefix_prefill_bf16pv", st)
    elif _uint8w:
        st = lib.i8kv_prefix_prefill_uint8w(*common, int(w_group), *tail)
        _raise("prefix_prefill_uint8w", st)
    else:
        st = lib.i8kv_prefix_prefill_int8(*common, int(w_group), *tail)
        _raise("prefix_prefill_int8", st)
    return out


@_allocates_on_stream
def prefix_prefill_ex(desc: CacheDesc, q_int8, q_scale, query_start_loc, seq_lens,
                      cache: PagedCache, block_tables, max_query_len: int, pv: str = "int8",
                      w_group: int = 32, out_bf16: bool = False,
                      softmax_scale: Optional[float] = None, out=None, stream=None):
    """The prefill with options: the PV variant ("int8", "bf16", "uint8") and a
    bf16 output (returned as torch.bfloat16); otherwise as prefix_prefill_int8."""
    import torch
    lib = load_library()
    Tq = int(q_int8.shape[0])
    S = int(seq_lens.shape[0])
    Hq, D = desc.num_q_heads, desc.head_dim
    _check(q_int8, "q_int8", torch.int8, (Tq, Hq, D))
    _check(q_scale, "q_scale", torch.float32, (Tq, Hq))
    _check(query_start_loc, "query_start_loc", torch.int32, (S + 1,))
    _check(seq_lens, "seq_lens", torch.int32, (S,))
    cache.check(desc)
    _check(block_tables, "block_tables", torch.int32)
    if block_tables.dim() != 2 or block_tables.shape[0] != S:
        raise ValueError(f"block_tables: shape {tuple(block_tables.shape)}, expected ({S}, *)")
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    if pv not in PV_VARIANTS:
        raise ValueError(f"pv must be one of {sorted(PV_VARIANTS)}")
    opts = PrefillOpts(int(w_group), float(softmax_scale), PV_VARIANTS[pv], 1 if out_bf16 else 0)
    dt = torch.bfloat16 if out_bf16 else torch.float32
    if out is None:
        out = torch.empty((Tq, Hq, D), dtype=dt, device=q_int8.device)
    _check(out, "out", dt, (Tq, Hq, D))
    st = lib.i8kv_prefix_prefill_ex(
        C.byref(desc), C.byref(opts), S, Tq, int(max_query_len), _ptr(q_int8), _ptr(q_scale),
        _ptr(query_start_loc), _ptr(seq_lens), _ptr(cache.k_cache), _ptr(cache.v_cache),
        _ptr(cache.k_scale), _ptr(cache.v_scale), _ptr(block_tables), int(block_tables.shape[1]),
        _ptr(out), _stream(stream))
    _raise("prefix_prefill_ex", st)
    return out


@_allocates_on_stream
def prefix_prefill_uint8w(desc: CacheDesc, q_int8, q_scale, query_start_loc, seq_lens,
                          cache: PagedCache, block_tables, max_query_len: int, w_group: int = 32,
                          softmax_scale: Optional[float] = None, out=None, workspace=None,
                          stream=None):
    """The UINT8-W variant of prefix_prefill_int8 (W groups quantized to
    0..255 against max W / 255); same arguments."""
    return prefix_prefill_int8(desc, q_int8, q_scale, query_start_loc, seq_lens, cache,
                               block_tables, max_query_len, w_group=w_group,
                               softmax_scale=softmax_scale, out=out, workspace=workspace,
                               stream=stream, _uint8w=True)


@_allocates_on_stream
def prefix_prefill_bf16pv(desc: CacheDesc, q_int8, q_scale, query_start_loc, seq_lens,
                          cache: PagedCache, block_tables, max_query_len: int,
                          softmax_scale: Optional[float] = None, out=None, workspace=None,
                          stream=None):
    """The BF16-PV ablation of prefix_prefill_int8 (same arguments without
    w_group)."""
    return prefix_prefill_int8(desc, q_int8, q_scale, query_start_loc, seq_lens, cache,
                               block_tables, max_query_len, softmax_scale=softmax_scale,
                               out=out, workspace=workspace, stream=stream, _bf16pv=True)


@_allocates_on_stream
def prefix_prefill_bf16qk(desc: CacheDesc, query, query_start_loc, seq_lens, cache: PagedCache,
                          block_tables, max_query_len: int, w_group: int = 32,
                          softmax_scale: Optional[float] = None, out=None, workspace=None,
                          stream=None):
    """The BF16-QK ablation of prefix_prefill_int8: ``query`` [total_q, Hq, D]
    bf16 (torch.bfloat16, or its bits as int16 / uint16), not quantized;
    the other arguments as prefix_prefill_int8."""
    import torch
    lib = load_library()
    Tq = int(query.shape[0])
    S = int(seq_lens.shape[0])
    Hq, D = desc.num_q_heads, desc.head_dim
    _check(query, "query", (torch.bfloat16, torch.int16, torch.uint16), (Tq, Hq, D))
    _check(query_start_loc, "query_start_loc", torch.int32, (S + 1,))
    _check(seq_lens, "seq_lens", torch.int32, (S,))
    cache.check(desc)
    _check(block_tables, "block_tables", torch.int32)
    if block_tables.dim() != 2 or block_tables.shape[0] != S:
        raise ValueError(f"block_tables: shape {tuple(block_tables.shape)}, expected ({S}, *)")
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((Tq, Hq, D), dtype=torch.float32, device=query.device)
    _check(out, "out", torch.float32, (Tq, Hq, D))
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.i8kv_prefix_prefill_bf16qk(
        C.byref(desc), S, Tq, int(max_query_len), _ptr(query), _ptr(query_start_loc),
        _ptr(seq_lens), _ptr(cache.k_cache), _ptr(cache.v_cache), _ptr(cache.k_scale),
        _ptr(cache.v_scale), _ptr(block_tables), int(block_tables.shape[1]), int(w_group),
        float(softmax_scale), _ptr(workspace), int(ws_bytes), _ptr(out), _stream(stream))
    _raise("prefix_prefill_bf16qk", st)
    return out
