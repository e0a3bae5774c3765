"""GPU parity of paged decode against the oracle.

The int8 caches must be bit-identical first (they feed both sides); decode
outputs must then agree with the oracle within max-abs 1e-3 and mean-abs
1e-4.  The error against unquantized fp64 attention is reported alongside.
"""
import numpy as np
import pytest

import workloads as W
from gpu_helpers import (assert_bits_equal, assert_close, cache_to_np, decode_queries, dev,
                         gpu_fill, report_fp64, say)
from refmath import decode_reference_fp64

pytestmark = pytest.mark.gpu


def run_decode(wl, orc, G, report=True, repeat=2):
    import int8_kv_quantized_amd as K
    say(f"  decode case {wl.name}: S={wl.num_seqs} Lmax={wl.max_seq_len} Hq={wl.num_q_heads} "
        f"Hkv={wl.num_kv_heads} D={wl.head_dim} G={G}")
    d, cache, q8, qs = gpu_fill(wl)
    ocache, oq8, oqs = orc.fill(wl)
    g = cache_to_np(cache)
    for k in g:
        assert_bits_equal(g[k], ocache[k], f"{wl.name} {k}")
    dq8, dqs = decode_queries(q8, qs, wl)
    bt, sl = dev(wl.block_tables), dev(wl.seq_lens)
    import torch
    ws = torch.zeros(max(256, K.paged_decode_workspace_bytes(d, wl.num_seqs, wl.max_seq_len)),
                     dtype=torch.uint8, device="cuda")
    outs = []
    for _ in range(repeat):
        out = K.paged_decode_int8(d, dq8, dqs, cache, bt, sl, wl.max_seq_len, w_group=G,
                                  workspace=ws)
        torch.cuda.synchronize()
        outs.append(out.cpu().numpy())
    rows = wl.decode_query_rows()
    ref = orc.paged_decode(oq8[rows], oqs[rows], ocache, wl.block_tables, wl.seq_lens,
                           num_q_heads=wl.num_q_heads, w_group=G)
    assert_close(outs[0], ref, f"{wl.name} G={G}")
    for o in outs[1:]:   # a second call over the same workspace gives the same bits
        assert np.array_equal(o, outs[0]), "repeated call differs"
    if report:
        report_fp64(outs[0], decode_reference_fp64(wl), f"{wl.name} G={G}")
    return outs[0], ref


SMALL = [
    dict(name="ragged_d128_g3", seq_lens=(37, 300, 16, 1, 700, 256, 257), num_q_heads=6,
         num_kv_heads=2, head_dim=128),
    dict(name="d64_mha", seq_lens=(5, 70, 513), num_q_heads=4, num_kv_heads=4, head_dim=64),
    dict(name="d256_g6", seq_lens=(33, 1024, 2000), num_q_heads=24, num_kv_heads=4,
         head_dim=256),
    dict(name="d256_g16", seq_lens=(40, 4000), num_q_heads=16, num_kv_heads=1, head_dim=256),
    dict(name="d128_g8_long", seq_lens=(9000,), num_q_heads=8, num_kv_heads=1, head_dim=128),
]


@pytest.mark.parametrize("G", [32, 64])
@pytest.mark.parametrize("kw", SMALL, ids=lambda k: k["name"])
def test_decode_small(orc, kw, G):
    kw = dict(kw)
    name = kw.pop("name")
    wl = W.make_workload(name, new_tokens=[1] * len(kw["seq_lens"]), seed=51, w_group=G, **kw)
    run_decode(wl, orc, G)


def test_decode_empty_sequence(orc):
    import int8_kv_quantized_amd as K
    import torch
    wl = W.make_workload("empty", seq_lens=[20, 300], new_tokens=[1, 1], num_q_heads=6,
                         num_kv_heads=2, head_dim=128, seed=52)
    say("  decode case empty: one sequence of length 0")
    d, cache, q8, qs = gpu_fill(wl)
    dq8, dqs = decode_queries(q8, qs, wl)
    lens = np.array([0, 300], np.int32)
    out = K.paged_decode_int8(d, dq8, dqs, cache, dev(wl.block_tables), dev(lens), 300)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    ocache, oq8, oqs = orc.fill(wl)
    rows = wl.decode_query_rows()
    ref = orc.paged_decode(oq8[rows], oqs[rows], ocache, wl.block_tables, lens, num_q_heads=6)
    assert not out[0].any()
    assert_close(out, ref, "empty")


@pytest.mark.parametrize("G", [32, 64])
def test_decode_zero_vectors(orc, G):
    """All-zero query vectors (sQ = 0: uniform softmax over the sequence) and
    all-zero key / value vectors (scale 0)."""
    wl = W.make_workload("zero_vectors", seq_lens=(700, 300, 40), new_tokens=[1, 1, 1],
                         num_q_heads=6, num_kv_heads=2, head_dim=128, seed=53, w_group=G)
    wl.query[0] = 0              # every head of the first sequence's query
    wl.query[1, 3] = 0           # one head of the second
    wl.key[::9, 0] = 0
    wl.value[5::17, 1] = 0
    run_decode(wl, orc, G)


@pytest.mark.parametrize("G", [32])
def test_decode_cfg1_L512(orc, G):
    run_decode(W.cfg1_decode_512(G), orc, G)


@pytest.mark.parametrize("G", [32, 64])
@pytest.mark.parametrize("L", [4096, 8192, 16384])
def test_decode_cfg2_outlier_v(orc, L, G):
    run_decode(W.cfg2_decode(L, G), orc, G)


def test_decode_cfg3_32k(orc):
    run_decode(W.cfg3_decode_32k(), orc, 32)


def test_decode_cfg3_batch16(orc):
    run_decode(W.cfg3_decode_batch16(), orc, 32, report=False)


@pytest.mark.parametrize("G", [32, 64])
def test_decode_cfg5_mha(orc, G):
    run_decode(W.cfg5_mha_producer_decode(G), orc, G)


def test_decode_many_sequences(orc):
    """700 sequences of seeded lengths 1 .. 700 (one to three partitions):
    700 workgroup rows in the grid of both kernels, every length class."""
    rng = np.random.default_rng(71)
    lens = rng.integers(1, 701, 700)
    wl = W.make_workload("many_seqs", seq_lens=tuple(int(x) for x in lens),
                         new_tokens=[1] * lens.size, num_q_heads=8, num_kv_heads=2, head_dim=128,
                         seed=71)
    run_decode(wl, orc, 32, report=False)


@pytest.mark.parametrize("G", [32, 64])
@pytest.mark.parametrize("shape", [(4, 2, 64), (8, 4, 256), (12, 4, 256), (16, 1, 256)],
                         ids=["d64_g2", "d256_g2", "d256_g3", "d256_g16"])
def test_decode_batch_of_rounds(orc, shape, G):
    """Grids of several rounds for every head size (60 sequences of seeded
    lengths 1 .. 3000, so most partition workgroups lie past their sequence
    and leave on the length): D = 64 and 256 with partials under 4 KB per
    workgroup (ordinary stores), D = 256 with three heads per KV head (the
    partials staged in LDS and stored non-temporally), and D = 256 with 16
    heads per KV head (the largest staged block, 16 rows x 256 dims)."""
    Hq, Hkv, D = shape
    rng = np.random.default_rng(73)
    lens = rng.integers(1, 3001, 60)
    wl = W.make_workload(f"rounds_{Hq}_{Hkv}_{D}", seq_lens=tuple(int(x) for x in lens),
                         new_tokens=[1] * lens.size, num_q_heads=Hq, num_kv_heads=Hkv,
                         head_dim=D, seed=73, w_group=G)
    assert ((int(lens.max()) + 255) // 256) * Hkv * lens.size > 256
    run_decode(wl, orc, G, report=False)


def test_decode_long_sequences_many_merge_rounds(orc):
    """150001 and 70000 tokens: 586 and 274 partitions, so the merge runs
    ten and five rounds of 64 partitions, with ragged last partitions."""
    wl = W.make_workload("long_decode", seq_lens=(150001, 70000), new_tokens=(1, 1),
                         num_q_heads=4, num_kv_heads=1, head_dim=64, seed=69)
    run_decode(wl, orc, 32, report=False)


def test_decode_max_length(orc):
    """The longest supported sequence, 2^20 tokens (4096 partitions: the merge
    runs 64 rounds), next to a ragged one 17 tokens shorter."""
    wl = W.make_workload("max_len_decode", seq_lens=((1 << 20), (1 << 20) - 17), new_tokens=(1, 1),
                         num_q_heads=2, num_kv_heads=1, head_dim=64, seed=70)
    run_decode(wl, orc, 32, report=False)
