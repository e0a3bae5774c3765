"""The decode's two stages as separate calls (i8kv_paged_decode_partials,
i8kv_paged_decode_merge).

* partials + merge over one workspace equal i8kv_paged_decode_int8 bit for
  bit (ragged batch with empty, one-partition and many-partition sequences),
  and the oracle within max-abs 1e-3, mean-abs 1e-4;
* a decode sharded over the partitions of one sequence: the sequence is cut
  at a multiple of 256 tokens into shards, each shard a sequence of its own
  whose block table starts at its first page; the shards' partials, placed
  in one workspace at their partition offsets, merge to the unsharded call's
  output bit for bit ([PV] 2.2: partitions are reduced independently and
  merged with log-sum-exp weights, so where a partition is computed does
  not matter).
"""
import numpy as np
import pytest

import workloads as W
from gpu_helpers import assert_bits_equal, assert_close, decode_queries, dev, gpu_fill, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("G", [32, 64])
def test_partials_then_merge_equal_the_call(orc, G):
    import int8_kv_quantized_amd as K
    import torch
    wl = W.make_workload("stages_ragged", seq_lens=(300, 1, 256, 1000, 257, 4096, 40),
                         new_tokens=[1] * 7, num_q_heads=24, num_kv_heads=4, head_dim=256,
                         seed=98, w_group=G)
    say(f"  stages case {wl.name} G={G}")
    d, cache, q8, qs = gpu_fill(wl)
    dq8, dqs = decode_queries(q8, qs, wl)
    lens = wl.seq_lens.astype(np.int32).copy()
    lens[1] = 0  # an empty sequence
    bt, sl, L = dev(wl.block_tables), dev(lens), wl.max_seq_len
    nbytes = K.paged_decode_workspace_bytes(d, wl.num_seqs, L)
    ws = torch.full(((nbytes + 3) // 4,), float("nan"), dtype=torch.float32, device="cuda")
    one = K.paged_decode_int8(d, dq8, dqs, cache, bt, sl, L, w_group=G)
    K.paged_decode_partials(d, dq8, dqs, cache, bt, sl, L, w_group=G, workspace=ws)
    two = K.paged_decode_merge(d, sl, L, ws)
    torch.cuda.synchronize()
    one, two = one.cpu().numpy(), two.cpu().numpy()
    assert_bits_equal(two, one, "partials + merge vs one call")
    assert not two[1].any(), "empty sequence must give zeros"
    ocache, oq8, oqs = orc.fill(wl)
    rows = wl.decode_query_rows()
    ref = orc.paged_decode(oq8[rows], oqs[rows], ocache, wl.block_tables, lens,
                           num_q_heads=wl.num_q_heads, w_group=G)
    assert_close(two, ref, f"{wl.name} G={G} stages")


@pytest.mark.parametrize("G", [32, 64])
def test_batched_call_equals_one_call_per_sequence(orc, G):
    """A batch of eight sequences (empty, one-partition and up to 128-partition
    ones) against each sequence decoded alone: bit for bit.  Alone, a
    sequence of more than 64 partitions is merged in 128-partition rounds,
    in the batch in 64-partition rounds; every lane adds its partitions in
    the same order either way.  The batch's partials + merge equal the batched
    call, and the oracle agrees within tolerance."""
    import int8_kv_quantized_amd as K
    import torch
    wl = W.make_workload("batch_vs_alone", seq_lens=(20000, 1, 256, 32768, 257, 9000, 600, 31000),
                         new_tokens=[1] * 8, num_q_heads=24, num_kv_heads=4, head_dim=256,
                         seed=96, w_group=G)
    say(f"  batch vs one call per sequence {wl.name} G={G}")
    d, cache, q8, qs = gpu_fill(wl)
    dq8, dqs = decode_queries(q8, qs, wl)
    lens = wl.seq_lens.astype(np.int32).copy()
    lens[4] = 0  # an empty sequence
    bt, sl, L = dev(wl.block_tables), dev(lens), wl.max_seq_len
    one = K.paged_decode_int8(d, dq8, dqs, cache, bt, sl, L, w_group=G)
    nbytes = K.paged_decode_workspace_bytes(d, wl.num_seqs, L)
    ws = torch.full(((nbytes + 3) // 4,), float("nan"), dtype=torch.float32, device="cuda")
    K.paged_decode_partials(d, dq8, dqs, cache, bt, sl, L, w_group=G, workspace=ws)
    two = K.paged_decode_merge(d, sl, L, ws)
    alone = []
    for i in range(wl.num_seqs):
        Li = max(int(lens[i]), 1)
        alone.append(K.paged_decode_int8(d, dq8[i:i + 1].contiguous(), dqs[i:i + 1].contiguous(),
                                         cache, dev(wl.block_tables[i:i + 1]), dev(lens[i:i + 1]),
                                         Li, w_group=G))
    torch.cuda.synchronize()
    one, two = one.cpu().numpy(), two.cpu().numpy()
    alone = np.concatenate([x.cpu().numpy() for x in alone])
    assert_bits_equal(one, alone, "batched call vs one call per sequence")
    assert_bits_equal(two, one, "partials + merge vs the call")
    assert not one[4].any(), "empty sequence must give zeros"
    ocache, oq8, oqs = orc.fill(wl)
    rows = wl.decode_query_rows()
    ref = orc.paged_decode(oq8[rows], oqs[rows], ocache, wl.block_tables, lens,
                           num_q_heads=wl.num_q_heads, w_group=G)
    assert_close(one, ref, f"{wl.name} G={G}")


def test_partials_then_merge_equal_the_call_32k(orc):
    """One 32768-token sequence: 128 partitions, merged in one 128-partition
    round (the batch-1 merge); the merge alone equals the call bit for bit."""
    import int8_kv_quantized_amd as K
    import torch
    wl = W.cfg3_decode_32k()
    say(f"  stages case {wl.name}")
    d, cache, q8, qs = gpu_fill(wl)
    dq8, dqs = decode_queries(q8, qs, wl)
    bt, sl, L = dev(wl.block_tables), dev(wl.seq_lens), wl.max_seq_len
    nbytes = K.paged_decode_workspace_bytes(d, wl.num_seqs, L)
    ws = torch.full(((nbytes + 3) // 4,), float("nan"), dtype=torch.float32, device="cuda")
    one = K.paged_decode_int8(d, dq8, dqs, cache, bt, sl, L, w_group=32)
    K.paged_decode_partials(d, dq8, dqs, cache, bt, sl, L, w_group=32, workspace=ws)
    two = K.paged_decode_merge(d, sl, L, ws)
    torch.cuda.synchronize()
    one, two = one.cpu().numpy(), two.cpu().numpy()
    assert_bits_equal(two, one, "partials + merge vs one call (32K)")
    ocache, oq8, oqs = orc.fill(wl)
    rows = wl.decode_query_rows()
    ref = orc.paged_decode(oq8[rows], oqs[rows], ocache, wl.block_tables, wl.seq_lens,
                           num_q_heads=wl.num_q_heads, w_group=32)
    assert_close(two, ref, f"{wl.name} stages")


@pytest.mark.parametrize("cuts", [(4096,), (2048, 8192, 12288)], ids=["2shards", "4shards"])
def test_decode_sharded_over_partitions(orc, cuts):
    """16384 tokens (the 16K configuration) cut into shards at multiples of 256."""
    import int8_kv_quantized_amd as K
    import torch
    wl = W.cfg2_decode(16384, 32)
    say(f"  sharded decode {wl.name} cuts={cuts}")
    d, cache, q8, qs = gpu_fill(wl)
    dq8, dqs = decode_queries(q8, qs, wl)
    L = int(wl.seq_lens[0])
    bt_full = wl.block_tables
    full = K.paged_decode_int8(d, dq8, dqs, cache, dev(bt_full), dev(wl.seq_lens), L)
    edges = [0, *cuts, L]
    P = -(-L // 256)
    nbytes = K.paged_decode_workspace_bytes(d, 1, L)
    ws = torch.full(((nbytes + 3) // 4,), float("nan"), dtype=torch.float32, device="cuda")
    Hkv, grp, D = d.num_kv_heads, d.group, d.head_dim
    o_all = ws[:Hkv * P * grp * D].view(Hkv, P, grp, D)
    ml_off = ((Hkv * P * grp * D * 4 + 255) // 256 * 256) // 4
    ml_all = ws[ml_off:ml_off + Hkv * P * grp * 2].view(Hkv, P, grp, 2)
    for a, b in zip(edges[:-1], edges[1:]):
        n = b - a
        p0, ps = a // 256, -(-n // 256)
        bt = np.ascontiguousarray(bt_full[:, a // 16:])
        sws = K.paged_decode_partials(d, dq8, dqs, cache, dev(bt), dev(np.array([n], np.int32)),
                                      n)
        o_s = sws.view(torch.float32)[:Hkv * ps * grp * D].view(Hkv, ps, grp, D)
        soff = ((Hkv * ps * grp * D * 4 + 255) // 256 * 256) // 4
        ml_s = sws.view(torch.float32)[soff:soff + Hkv * ps * grp * 2].view(Hkv, ps, grp, 2)
        o_all[:, p0:p0 + ps].copy_(o_s)       # the exchange of partials
        ml_all[:, p0:p0 + ps].copy_(ml_s)
    merged = K.paged_decode_merge(d, dev(wl.seq_lens), L, ws)
    torch.cuda.synchronize()
    assert_bits_equal(merged.cpu().numpy(), full.cpu().numpy(), f"sharded {cuts} vs one call")
