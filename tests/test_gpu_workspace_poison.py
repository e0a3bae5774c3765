"""The decode workspace needs no initialization.

Every decode entry point is run over a workspace filled with NaN, then with
+Inf, and compared with the oracle (max-abs 1e-3, mean-abs 1e-4).  The cases
are the ones where the merge meets workspace slots that the partition kernel
never writes: ragged batches (a short sequence next to a long one), a batch-1
call whose max_seq_len lies several partitions past seq_lens[0], several
queries per sequence, the fused step, every PV/QK variant, and a batch-1
call long enough for the merge's 128-partition rounds.  The merge of
partition outputs with log-sum-exp weights follows the page "Implementing
INT8 PV MMAC on a gfx936 DCU", section 2.2: only a sequence's own partitions
enter its sum.
"""
import numpy as np
import pytest

import workloads as W
from gpu_helpers import (assert_bits_equal, assert_close, cache_to_np, decode_queries, desc_of,
                         dev, gpu_fill, say, split_tokens)

pytestmark = pytest.mark.gpu

FILLS = {"nan": float("nan"), "inf": float("inf")}


def poisoned(nbytes, fill):
    import torch
    n = (max(256, int(nbytes)) + 3) // 4
    return torch.full((n,), FILLS[fill], dtype=torch.float32, device="cuda")


def past_end(wl, extra_parts):
    """max_seq_len of the call: the longest sequence plus extra partitions."""
    return int(wl.max_seq_len) + 256 * extra_parts


def ragged_small(G=32, **kw):
    return W.make_workload("poison_ragged", seq_lens=(300, 5, 1000, 256, 17), new_tokens=[1] * 5,
                           num_q_heads=6, num_kv_heads=2, head_dim=128, seed=91, w_group=G, **kw)


def batch1_short(G=32):
    return W.make_workload("poison_batch1", seq_lens=(700,), new_tokens=(1,), num_q_heads=24,
                           num_kv_heads=4, head_dim=256, seed=92, w_group=G)


def batch1_long(G=32):
    """67 partitions: a batch-1 call with more than 64 partitions merges 128 per
    round, whose first round loads slots 67 .. 127 before the length is known."""
    return W.make_workload("poison_batch1_long", seq_lens=(17000,), new_tokens=(1,),
                           num_q_heads=24, num_kv_heads=4, head_dim=256, seed=97, w_group=G)


def decode_case(wl, orc, fill, G=32, extra_parts=0):
    import int8_kv_quantized_amd as K
    import torch
    L = past_end(wl, extra_parts)
    say(f"  poisoned ({fill}) decode {wl.name}: S={wl.num_seqs} max_seq_len={L} G={G}")
    d, cache, q8, qs = gpu_fill(wl)
    dq8, dqs = decode_queries(q8, qs, wl)
    bt = np.zeros((wl.num_seqs, -(-L // 16)), np.int32)
    bt[:, :wl.block_tables.shape[1]] = wl.block_tables
    ws = poisoned(K.paged_decode_workspace_bytes(d, wl.num_seqs, L), fill)
    out = K.paged_decode_int8(d, dq8, dqs, cache, dev(bt), dev(wl.seq_lens), L, w_group=G,
                              workspace=ws)
    torch.cuda.synchronize()
    ocache, oq8, oqs = orc.fill(wl)
    rows = wl.decode_query_rows()
    ref = orc.paged_decode(oq8[rows], oqs[rows], ocache, wl.block_tables, wl.seq_lens,
                           num_q_heads=wl.num_q_heads, w_group=G)
    assert_close(out.cpu().numpy(), ref, f"{wl.name} poisoned {fill}")


@pytest.mark.parametrize("fill", list(FILLS))
def test_poisoned_cfg3_batch16(orc, fill):
    decode_case(W.cfg3_decode_batch16(), orc, fill)


@pytest.mark.parametrize("fill", list(FILLS))
@pytest.mark.parametrize("G", [32, 64])
def test_poisoned_cfg5_mha(orc, fill, G):
    decode_case(W.cfg5_mha_producer_decode(G), orc, fill, G=G)


@pytest.mark.parametrize("fill", list(FILLS))
@pytest.mark.parametrize("G", [32, 64])
def test_poisoned_batch1_max_len_past_sequence(orc, fill, G):
    decode_case(batch1_short(G), orc, fill, G=G, extra_parts=5)


@pytest.mark.parametrize("fill", list(FILLS))
def test_poisoned_batch1_long_two_merge_rounds(orc, fill):
    """max_seq_len 70 partitions past the sequence: 137 workspace slots, two
    128-partition merge rounds, every slot from 67 on never written."""
    decode_case(batch1_long(), orc, fill, extra_parts=70)


@pytest.mark.parametrize("fill", list(FILLS))
def test_poisoned_ragged_max_len_past_sequences(orc, fill):
    decode_case(ragged_small(), orc, fill, extra_parts=3)


@pytest.mark.parametrize("fill", list(FILLS))
def test_poisoned_decode_ex_8_queries(orc, fill):
    import int8_kv_quantized_amd as K
    import torch
    from test_gpu_decode_ex import multi_queries
    nq = 8
    wl = W.make_workload("poison_ex", seq_lens=(700, 9, 300, 1200), new_tokens=[nq] * 4,
                         num_q_heads=4, num_kv_heads=4, head_dim=128, seed=93)
    L = past_end(wl, 2)
    say(f"  poisoned ({fill}) decode_ex nq={nq} {wl.name}: max_seq_len={L}")
    d, cache, q8, qs = gpu_fill(wl)
    q8m, qsm = multi_queries(q8.cpu().numpy(), qs.cpu().numpy(), wl, nq)
    bt = np.zeros((wl.num_seqs, -(-L // 16)), np.int32)
    bt[:, :wl.block_tables.shape[1]] = wl.block_tables
    opts = K.DecodeOpts(256, 32, float(np.float32(1 / np.sqrt(128))), 0, nq, 0)
    ws = poisoned(K.paged_decode_ex_workspace_bytes(d, opts, wl.num_seqs, L), fill)
    out = K.paged_decode_ex(d, dev(q8m), dev(qsm), cache, dev(bt), dev(wl.seq_lens), L,
                            queries_per_seq=nq, workspace=ws)
    torch.cuda.synchronize()
    ocache, _, _ = orc.fill(wl)
    ref = orc.paged_decode_multi(q8m, qsm, ocache, wl.block_tables, wl.seq_lens,
                                 num_q_heads=wl.num_q_heads, queries_per_seq=nq)
    assert_close(out.cpu().numpy(), ref, f"{wl.name} poisoned {fill}")


@pytest.mark.parametrize("fill", list(FILLS))
def test_poisoned_fused_step(orc, fill):
    import int8_kv_quantized_amd as K
    import torch
    wl = ragged_small()
    L = past_end(wl, 3)
    say(f"  poisoned ({fill}) fused step {wl.name}: max_seq_len={L}")
    d = desc_of(wl)
    hist, qi = split_tokens(wl)
    rows = wl.decode_query_rows()
    newest = qi[rows]
    cache = K.PagedCache.allocate(d)
    K.kv_quantize_write(d, dev(wl.key[hist]), dev(wl.value[hist]), dev(wl.slot_mapping[hist]),
                        cache)
    bt = np.zeros((wl.num_seqs, -(-L // 16)), np.int32)
    bt[:, :wl.block_tables.shape[1]] = wl.block_tables
    ws = poisoned(K.paged_decode_workspace_bytes(d, wl.num_seqs, L), fill)
    out = K.decode_step_int8(d, dev(wl.key[newest]), dev(wl.value[newest]), dev(wl.query[rows]),
                             cache, dev(bt), dev(wl.seq_lens), L, workspace=ws)
    torch.cuda.synchronize()
    ocache, oq8, oqs = orc.fill(wl)
    g = cache_to_np(cache)
    for k in g:
        assert_bits_equal(g[k], ocache[k], f"{wl.name} fused {k}")
    ref = orc.paged_decode(oq8[rows], oqs[rows], ocache, wl.block_tables, wl.seq_lens,
                           num_q_heads=wl.num_q_heads)
    assert_close(out.cpu().numpy(), ref, f"{wl.name} fused poisoned {fill}")


@pytest.mark.parametrize("fill", list(FILLS))
@pytest.mark.parametrize("variant", ["bf16pv", "uint8w", "bf16qk"])
def test_poisoned_variants(orc, fill, variant):
    import int8_kv_quantized_amd as K
    import oracle
    import torch
    wl = ragged_small()
    L = past_end(wl, 3)
    say(f"  poisoned ({fill}) {variant} decode {wl.name}: max_seq_len={L}")
    d, cache, q8, qs = gpu_fill(wl)
    dq8, dqs = decode_queries(q8, qs, wl)
    bt = np.zeros((wl.num_seqs, -(-L // 16)), np.int32)
    bt[:, :wl.block_tables.shape[1]] = wl.block_tables
    bt, sl = dev(bt), dev(wl.seq_lens)
    ws = poisoned(K.paged_decode_workspace_bytes(d, wl.num_seqs, L), fill)
    ocache, oq8, oqs = orc.fill(wl)
    rows = wl.decode_query_rows()
    if variant == "bf16pv":
        out = K.paged_decode_bf16pv(d, dq8, dqs, cache, bt, sl, L, workspace=ws)
        ref = orc.paged_decode(oq8[rows], oqs[rows], ocache, wl.block_tables, wl.seq_lens,
                               num_q_heads=wl.num_q_heads, flags=oracle.ORC_BF16_PV)
    elif variant == "uint8w":
        out = K.paged_decode_uint8w(d, dq8, dqs, cache, bt, sl, L, workspace=ws)
        ref = orc.paged_decode(oq8[rows], oqs[rows], ocache, wl.block_tables, wl.seq_lens,
                               num_q_heads=wl.num_q_heads, flags=oracle.ORC_UINT8_W)
    else:
        qb = np.ascontiguousarray(wl.query[rows])
        out = K.paged_decode_bf16qk(d, dev(qb.view(np.int16)), cache, bt, sl, L, workspace=ws)
        ref = orc.paged_decode_bf16qk(qb, ocache, wl.block_tables, wl.seq_lens)
    torch.cuda.synchronize()
    assert_close(out.cpu().numpy(), ref, f"{wl.name} {variant} poisoned {fill}")
