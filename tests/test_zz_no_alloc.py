"""i8kv_paged_decode_int8_noalloc: the decode with its partials in the
library's fixed per-GPU array instead of a caller workspace.

Called through the C ABI (ctypes, raw device pointers, a preallocated
output) and compared bit for bit with i8kv_paged_decode_int8 on the same
inputs -- the same kernels over the same workspace layout -- on two calls in a
row, the second with a smaller input (fewer sequences, shorter ones), so the
array holds the first call's partials when the second runs.  Sizes past the
array are rejected before any launch.  Also checked against the oracle
(max-abs 1e-3, mean-abs 1e-4).
"""
import ctypes as C

import numpy as np
import pytest

import workloads as W
from gpu_helpers import assert_bits_equal, assert_close, decode_queries, dev, gpu_fill, say

pytestmark = pytest.mark.gpu

WORKSPACE = 4


def noalloc_call(K, d, dq8, dqs, cache, bt, sl, L, G, out):
    import torch
    lib = K.load_library()
    P = lambda t: C.c_void_p(t.data_ptr())
    return lib.i8kv_paged_decode_int8_noalloc(
        C.byref(d), int(sl.shape[0]), P(dq8), P(dqs), P(cache.k_cache), P(cache.v_cache),
        P(cache.k_scale), P(cache.v_scale), P(bt), int(bt.shape[1]), P(sl), int(L), 256, int(G),
        float(np.float32(1.0 / np.sqrt(d.head_dim))),
        P(out), C.c_void_p(torch.cuda.current_stream().cuda_stream))


@pytest.mark.parametrize("G", [32, 64])
def test_noalloc_matches_workspace_call_twice(orc, G):
    import int8_kv_quantized_amd as K
    import torch
    cases = [
        W.make_workload("noalloc_big", seq_lens=(9000, 300, 4096, 1, 2500, 700), new_tokens=[1] * 6,
                        num_q_heads=24, num_kv_heads=4, head_dim=256, seed=101, w_group=G),
        W.make_workload("noalloc_small", seq_lens=(1000, 40), new_tokens=[1] * 2,
                        num_q_heads=24, num_kv_heads=4, head_dim=256, seed=102, w_group=G),
    ]
    for wl in cases:
        say(f"  no-alloc decode {wl.name}: S={wl.num_seqs} Lmax={wl.max_seq_len} G={G}")
        d, cache, q8, qs = gpu_fill(wl)
        dq8, dqs = decode_queries(q8, qs, wl)
        bt, sl, L = dev(wl.block_tables), dev(wl.seq_lens), wl.max_seq_len
        ref_gpu = K.paged_decode_int8(d, dq8, dqs, cache, bt, sl, L, w_group=G)
        out = torch.full((wl.num_seqs, d.num_q_heads, d.head_dim), float("nan"),
                         dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()
        st = noalloc_call(K, d, dq8, dqs, cache, bt, sl, L, G, out)
        assert st == 0, f"status {st}"
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        assert_bits_equal(got, ref_gpu.cpu().numpy(), f"{wl.name} no-alloc vs workspace call")
        ocache, oq8, oqs = orc.fill(wl)
        rows = wl.decode_query_rows()
        ref = orc.paged_decode(oq8[rows], oqs[rows], ocache, wl.block_tables, wl.seq_lens,
                               num_q_heads=wl.num_q_heads, w_group=G)
        assert_close(got, ref, f"{wl.name} G={G} no-alloc")


def test_noalloc_rejects_sizes_past_the_array():
    import int8_kv_quantized_amd as K
    import torch
    d = K.CacheDesc(24, 4, 256, 64)
    cap = K.paged_decode_noalloc_max_bytes()
    S, L = 32, 32768                  # 4096 partitions x 24 rows x (256 + 2) x 4 bytes
    assert K.paged_decode_workspace_bytes(d, S, L) > cap
    t = torch.zeros(16, dtype=torch.int32, device="cuda")
    lib = K.load_library()
    P = lambda x: C.c_void_p(x.data_ptr())
    st = lib.i8kv_paged_decode_int8_noalloc(C.byref(d), S, P(t), P(t), P(t), P(t), P(t), P(t),
                                            P(t), L // 16, P(t), L, 256, 32, 0.0625, P(t), None)
    assert st == WORKSPACE
    assert K.paged_decode_workspace_bytes(d, 16, 32768) <= cap
