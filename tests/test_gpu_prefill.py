"""GPU parity of chunked prefill with history against the oracle.

Small ragged cases compare every output.  The full 2048-over-16384 chunk is
compared on every one of its 2048 query rows and 24 heads (the oracle runs on
a host thread pool); the error against unquantized fp64 attention is reported
on the first and last row of every 32-row tile.  Tolerance: max-abs 1e-3,
mean-abs 1e-4, except that a W code whose quotient W / sW lies within 1e-4 of
a rounding tie may be decided either way (one code unit of that key's
contribution, sW |Vq| / l, on top of 1e-3 for that row; see
gpu_helpers.prefill_tie_allowance) -- with few keys per row (small l) one
such code alone can move an output past 1e-3.
"""
import numpy as np
import pytest

import workloads as W
from gpu_helpers import (assert_bits_equal, assert_close, assert_close_prefill, cache_to_np, dev,
                         gpu_fill, oracle_rows, prefill_tie_allowance, report_fp64,
                         row_tile_ends, say)
from refmath import prefill_reference_fp64

pytestmark = pytest.mark.gpu


def run_prefill(wl, orc, G, rows=None, fp64_rows=None):
    import int8_kv_quantized_amd as K
    import torch
    say(f"  prefill case {wl.name}: S={wl.num_seqs} Tq={wl.query.shape[0]} "
        f"Lmax={wl.max_seq_len} Hq={wl.num_q_heads} Hkv={wl.num_kv_heads} "
        f"D={wl.head_dim} G={G} rows={'all' if rows is None else len(rows)}")
    d, cache, q8, qs = gpu_fill(wl)
    ocache, oq8, oqs = orc.fill(wl)
    g = cache_to_np(cache)
    for k in g:
        assert_bits_equal(g[k], ocache[k], f"{wl.name} {k}")
    qsl = wl.query_start_loc
    max_q = int((qsl[1:] - qsl[:-1]).max())
    out = K.prefix_prefill_int8(d, q8, qs, dev(qsl), dev(wl.seq_lens), cache,
                                dev(wl.block_tables), max_q, w_group=G)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    r = np.arange(out.shape[0], dtype=np.int32) if rows is None else np.asarray(rows, np.int32)
    ref = oracle_rows(lambda **kw: orc.prefix_prefill(oq8, oqs, qsl, wl.seq_lens, ocache,
                                                      wl.block_tables, w_group=G, **kw),
                      r, np.zeros_like(out))
    say(f"    compared {r.size} query rows x {wl.num_q_heads} heads")
    tie = lambda row, head: prefill_tie_allowance(orc, oq8, oqs, qsl, wl.seq_lens, ocache,
                                                  wl.block_tables, row, head, G)
    assert_close_prefill(out[r], ref[r], r, tie, f"{wl.name} G={G}")
    r64 = r if fp64_rows is None else np.asarray(fp64_rows, np.int32)
    ref64 = prefill_reference_fp64(wl, rows=r64)
    report_fp64(out[r64], ref64[r64], f"{wl.name} G={G} ({r64.size} rows)")


SMALL = [
    dict(name="ragged_d128_g3", seq_lens=(40, 300, 33, 130, 700), new_tokens=(8, 50, 33, 1, 200),
         num_q_heads=6, num_kv_heads=2, head_dim=128),
    dict(name="d64_mha", seq_lens=(70, 129), new_tokens=(70, 64), num_q_heads=4, num_kv_heads=4,
         head_dim=64),
    dict(name="d256_g6", seq_lens=(600, 300), new_tokens=(100, 37), num_q_heads=24,
         num_kv_heads=4, head_dim=256),
    dict(name="d256_g16", seq_lens=(200,), new_tokens=(65,), num_q_heads=16, num_kv_heads=1,
         head_dim=256),
]


def test_prefill_many_sequences(orc):
    """200 sequences: seeded histories of 0 .. 400 tokens and chunks of 1 .. 24
    queries (200 workgroup planes in the grid; short and empty histories,
    chunks shorter than a row tile)."""
    rng = np.random.default_rng(72)
    chunks = rng.integers(1, 25, 200)
    hist = rng.integers(0, 401, 200)
    wl = W.make_workload("many_seqs_prefill", seed=72, kind="prefill",
                         seq_lens=tuple(int(h + c) for h, c in zip(hist, chunks)),
                         new_tokens=tuple(int(c) for c in chunks), num_q_heads=6,
                         num_kv_heads=2, head_dim=128, w_group=32)
    run_prefill(wl, orc, 32)


@pytest.mark.parametrize("G", [32, 64])
@pytest.mark.parametrize("kw", SMALL, ids=lambda k: k["name"])
def test_prefill_small(orc, kw, G):
    kw = dict(kw)
    name = kw.pop("name")
    wl = W.make_workload(name, seed=61, kind="prefill", w_group=G, **kw)
    run_prefill(wl, orc, G)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("G", [32, 64])
def test_prefill_cfg4_every_row(orc, G):
    """All 2048 x 24 outputs of the 2048-over-16384 chunk against the oracle."""
    wl = W.cfg4_prefill(w_group=G)
    run_prefill(wl, orc, G, fp64_rows=row_tile_ends(2048))


@pytest.mark.parametrize("G", [32, 64])
def test_prefill_zero_vectors(orc, G):
    """All-zero query vectors (sQ = 0: every visible score 0, a uniform softmax)
    and all-zero key / value vectors (scale 0) inside the chunk and history."""
    wl = W.make_workload("zero_vectors", seed=67, kind="prefill", w_group=G,
                         seq_lens=(150, 90), new_tokens=(70, 90), num_q_heads=6,
                         num_kv_heads=2, head_dim=128)
    wl.query[::5, :, :] = 0          # every fifth query token, all heads
    wl.query[1::7, 2, :] = 0         # one head of others
    wl.key[::11, 1, :] = 0           # some keys of KV head 1
    wl.value[3::13, 0, :] = 0        # some values of KV head 0
    run_prefill(wl, orc, G)


def test_prefill_history_beyond_lds_block_table(orc):
    """70000 history tokens = 4378 pages, more than the 4096 block-table
    entries the kernel caches in LDS: every page id is then read from the
    block table in global memory.  Sampled rows of a 40-token chunk."""
    wl = W.make_workload("history_70k", seed=68, kind="prefill", seq_lens=(70040,),
                         new_tokens=(40,), num_q_heads=2, num_kv_heads=1, head_dim=64)
    run_prefill(wl, orc, 32, rows=[0, 1, 17, 38, 39])
