"""Every entry point run on a side stream, with the binding allocating what
the call needs (workspace, outputs, quantized queries).

The side stream is first kept busy (a spin kernel), so the kernels of the call
are still queued when the binding returns and releases its workspace; a
tensor of the same size is then allocated and filled with NaN on the default
stream.  A workspace allocated on the wrong stream could be handed to that
tensor while the kernels still use it.  Results are compared with the oracle
(caches bit-exact, outputs max-abs 1e-3, mean-abs 1e-4).
"""
import numpy as np
import pytest

import workloads as W
from gpu_helpers import (assert_bits_equal, assert_close, cache_to_np, decode_queries, desc_of,
                         dev, gpu_fill, say, split_tokens)

pytestmark = pytest.mark.gpu


def busy_side_stream():
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    if hasattr(torch.cuda, "_sleep"):
        with torch.cuda.stream(s):
            torch.cuda._sleep(20_000_000)
    return s


def scribble(nbytes):
    """Allocate and NaN-fill a tensor on the default stream right after a call."""
    import torch
    return torch.full((max(64, int(nbytes) // 4),), float("nan"), dtype=torch.float32,
                      device="cuda")


def ragged(G=32):
    return W.make_workload("side_ragged", seq_lens=(300, 5, 1000, 256), new_tokens=[1] * 4,
                           num_q_heads=6, num_kv_heads=2, head_dim=128, seed=95, w_group=G)


def test_side_stream_producer(orc):
    import int8_kv_quantized_amd as K
    import torch
    wl = ragged()
    say(f"  side-stream producer {wl.name}")
    d = desc_of(wl)
    cache = K.PagedCache.allocate(d)
    s = busy_side_stream()
    q8, qs = K.kv_quantize_write(d, dev(wl.key), dev(wl.value), dev(wl.slot_mapping), cache,
                                 query=dev(np.repeat(wl.query[:1], wl.num_tokens, 0)), stream=s)
    junk = scribble(q8.numel())
    s.synchronize()
    torch.cuda.synchronize()
    ocache = orc.empty_cache(wl.num_blocks, wl.num_kv_heads, wl.head_dim)
    oq8, oqs = orc.kv_quantize_write(wl.key, wl.value, wl.slot_mapping, ocache,
                                     num_q_heads=wl.num_q_heads,
                                     query=np.repeat(wl.query[:1], wl.num_tokens, 0))
    g = cache_to_np(cache)
    for k in g:
        assert_bits_equal(g[k], ocache[k], f"side-stream {k}")
    assert_bits_equal(q8.cpu().numpy(), oq8, "side-stream q_int8")
    assert_bits_equal(qs.cpu().numpy(), oqs, "side-stream q_scale")
    del junk


@pytest.mark.parametrize("entry", ["int8", "uint8w", "bf16pv", "bf16qk", "ex_nq2", "step"])
def test_side_stream_decode(orc, entry):
    import int8_kv_quantized_amd as K
    import oracle
    import torch
    wl = ragged() if entry != "ex_nq2" else W.make_workload(
        "side_ex", seq_lens=(300, 5, 1000), new_tokens=[2] * 3, num_q_heads=6, num_kv_heads=2,
        head_dim=128, seed=96)
    say(f"  side-stream decode {entry} {wl.name}")
    d, cache, q8, qs = gpu_fill(wl)
    ocache, oq8, oqs = orc.fill(wl)
    rows = wl.decode_query_rows()
    dq8, dqs = decode_queries(q8, qs, wl)
    bt, sl, L = dev(wl.block_tables), dev(wl.seq_lens), wl.max_seq_len
    ws_bytes = K.paged_decode_workspace_bytes(d, wl.num_seqs, L)
    s = busy_side_stream()
    if entry == "int8":
        out = K.paged_decode_int8(d, dq8, dqs, cache, bt, sl, L, stream=s)
        ref = orc.paged_decode(oq8[rows], oqs[rows], ocache, wl.block_tables, wl.seq_lens,
                               num_q_heads=wl.num_q_heads)
    elif entry == "uint8w":
        out = K.paged_decode_uint8w(d, dq8, dqs, cache, bt, sl, L, stream=s)
        ref = orc.paged_decode(oq8[rows], oqs[rows], ocache, wl.block_tables, wl.seq_lens,
                               num_q_heads=wl.num_q_heads, flags=oracle.ORC_UINT8_W)
    elif entry == "bf16pv":
        out = K.paged_decode_bf16pv(d, dq8, dqs, cache, bt, sl, L, stream=s)
        ref = orc.paged_decode(oq8[rows], oqs[rows], ocache, wl.block_tables, wl.seq_lens,
                               num_q_heads=wl.num_q_heads, flags=oracle.ORC_BF16_PV)
    elif entry == "bf16qk":
        qb = np.ascontiguousarray(wl.query[rows])
        out = K.paged_decode_bf16qk(d, dev(qb.view(np.int16)), cache, bt, sl, L, stream=s)
        ref = orc.paged_decode_bf16qk(qb, ocache, wl.block_tables, wl.seq_lens)
    elif entry == "ex_nq2":
        from test_gpu_decode_ex import multi_queries
        q8m, qsm = multi_queries(q8.cpu().numpy(), qs.cpu().numpy(), wl, 2)
        out = K.paged_decode_ex(d, dev(q8m), dev(qsm), cache, bt, sl, L, queries_per_seq=2,
                                stream=s)
        ws_bytes *= 2
        ref = orc.paged_decode_multi(q8m, qsm, ocache, wl.block_tables, wl.seq_lens,
                                     num_q_heads=wl.num_q_heads, queries_per_seq=2)
    else:
        hist, qi = split_tokens(wl)
        newest = qi[rows]
        base = K.PagedCache.allocate(d)
        K.kv_quantize_write(d, dev(wl.key[hist]), dev(wl.value[hist]),
                            dev(wl.slot_mapping[hist]), base)
        key, value, query = dev(wl.key[newest]), dev(wl.value[newest]), dev(wl.query[rows])
        s = busy_side_stream()
        out = K.decode_step_int8(d, key, value, query, base, bt, sl, L, stream=s)
        ref = orc.paged_decode(oq8[rows], oqs[rows], ocache, wl.block_tables, wl.seq_lens,
                               num_q_heads=wl.num_q_heads)
    junk = scribble(ws_bytes)
    s.synchronize()
    torch.cuda.synchronize()
    assert_close(out.cpu().numpy(), ref, f"side-stream {entry}")
    del junk


@pytest.mark.parametrize("entry", ["int8", "bf16pv", "bf16qk"])
def test_side_stream_prefill(orc, entry):
    import int8_kv_quantized_amd as K
    import oracle
    import torch
    wl = W.make_workload("side_prefill", seed=97, kind="prefill", seq_lens=(300, 90),
                         new_tokens=(100, 37), num_q_heads=6, num_kv_heads=2, head_dim=128)
    say(f"  side-stream prefill {entry} {wl.name}")
    d, cache, q8, qs = gpu_fill(wl)
    ocache, oq8, oqs = orc.fill(wl)
    qsl = wl.query_start_loc
    loc = (dev(qsl), dev(wl.seq_lens), cache, dev(wl.block_tables), 100)
    s = busy_side_stream()
    if entry == "int8":
        out = K.prefix_prefill_int8(d, q8, qs, *loc, stream=s)
        ref = orc.prefix_prefill(oq8, oqs, qsl, wl.seq_lens, ocache, wl.block_tables)
    elif entry == "bf16pv":
        out = K.prefix_prefill_bf16pv(d, q8, qs, *loc, stream=s)
        ref = orc.prefix_prefill(oq8, oqs, qsl, wl.seq_lens, ocache, wl.block_tables, tile=64,
                                 flags=oracle.ORC_BF16_PV)
    else:
        out = K.prefix_prefill_bf16qk(d, dev(wl.query.view(np.int16)), *loc, stream=s)
        ref = orc.prefix_prefill_bf16qk(wl.query, qsl, wl.seq_lens, ocache, wl.block_tables)
    junk = scribble(out.numel() * 4)
    s.synchronize()
    torch.cuda.synchronize()
    assert_close(out.cpu().numpy(), ref, f"side-stream prefill {entry}")
    del junk
