"""GPU parity of the prefill BF16-QK ablation (the bf16 queries, not
quantized, against the int8 K codes converted to bf16 in LDS, on the bf16
matrix unit) against the oracle's orc_prefix_prefill_bf16qk: max-abs 1e-3,
mean-abs 1e-4.  A bf16 query that is int8 codes times 2^-6 reproduces the
int8 path with q_scale = 2^-6 bit for bit.  The error of both QK variants
against unquantized fp64 attention is reported."""
import numpy as np
import pytest

import workloads as W
from gpu_helpers import (assert_bits_equal, assert_close, cache_to_np, dev, gpu_fill,
                         oracle_rows, report_fp64, row_tile_ends, say)
from refmath import prefill_reference_fp64

pytestmark = pytest.mark.gpu


def run_prefill_bf16qk(wl, orc, G=32, rows=None):
    import torch

    import int8_kv_quantized_amd as K
    say(f"  bf16-QK prefill case {wl.name}: S={wl.num_seqs} Tq={wl.query.shape[0]} "
        f"Lmax={wl.max_seq_len} Hq={wl.num_q_heads} Hkv={wl.num_kv_heads} D={wl.head_dim} "
        f"G={G} rows={'all' if rows is None else len(rows)}")
    d, cache, q8, qs = gpu_fill(wl)
    ocache, oq8, oqs = orc.fill(wl)
    g = cache_to_np(cache)
    for k in g:
        assert_bits_equal(g[k], ocache[k], f"{wl.name} {k}")
    qsl = wl.query_start_loc
    max_q = int((qsl[1:] - qsl[:-1]).max())
    loc = (dev(qsl), dev(wl.seq_lens), cache, dev(wl.block_tables), max_q)
    out = K.prefix_prefill_bf16qk(d, dev(wl.query.view(np.int16)), *loc, w_group=G)
    out8 = K.prefix_prefill_int8(d, q8, qs, *loc, w_group=G)
    torch.cuda.synchronize()
    out, out8 = out.cpu().numpy(), out8.cpu().numpy()
    r = np.arange(out.shape[0], dtype=np.int32) if rows is None else np.asarray(rows, np.int32)
    ref = oracle_rows(lambda **kw: orc.prefix_prefill_bf16qk(wl.query, qsl, wl.seq_lens, ocache,
                                                             wl.block_tables, w_group=G, tile=64,
                                                             **kw),
                      r, np.zeros_like(out))
    say(f"    compared {r.size} query rows x {wl.num_q_heads} heads")
    sel = r
    assert_close(out[sel], ref[sel], f"{wl.name} bf16-QK G={G}")
    ref64 = prefill_reference_fp64(wl, rows=r)
    report_fp64(out[sel], ref64[sel], f"{wl.name} bf16-QK G={G}")
    report_fp64(out8[sel], ref64[sel], f"{wl.name} int8-QK G={G}")


SMALL = [
    dict(name="ragged_d128_g3", seq_lens=(40, 300, 33, 130, 700), new_tokens=(8, 50, 33, 1, 200),
         num_q_heads=6, num_kv_heads=2, head_dim=128),
    dict(name="d64_mha", seq_lens=(70, 129), new_tokens=(70, 64), num_q_heads=4, num_kv_heads=4,
         head_dim=64),
    dict(name="d256_g6", seq_lens=(600, 300), new_tokens=(100, 37), num_q_heads=24,
         num_kv_heads=4, head_dim=256),
    dict(name="d256_g8_rows_past_chunk", seq_lens=(45,), new_tokens=(45,), num_q_heads=8,
         num_kv_heads=1, head_dim=256),
]


@pytest.mark.parametrize("G", [32, 64])
@pytest.mark.parametrize("kw", SMALL, ids=lambda k: k["name"])
def test_prefill_bf16qk_small(orc, kw, G):
    kw = dict(kw)
    name = kw.pop("name")
    wl = W.make_workload(name, seed=93, kind="prefill", **kw)
    run_prefill_bf16qk(wl, orc, G=G)


@pytest.mark.parametrize("D", [64, 128, 256])
def test_prefill_bf16qk_power_of_two_query_matches_int8_path(orc, D):
    """q = int8 codes * 2^-6 in bf16 against the int8 path with q_scale = 2^-6:
    bit-identical outputs."""
    import torch

    import int8_kv_quantized_amd as K
    wl = W.make_workload(f"pow2_d{D}", seq_lens=(300, 90), new_tokens=(120, 90), num_q_heads=8,
                         num_kv_heads=2, head_dim=D, seed=94, kind="prefill")
    say(f"  bf16-QK prefill power-of-two case D={D}")
    d, cache, q8, qs = gpu_fill(wl)
    qb = W.f32_to_bf16_bits(q8.cpu().numpy().astype(np.float32) * np.float32(2.0 ** -6))
    qsl = wl.query_start_loc
    max_q = int((qsl[1:] - qsl[:-1]).max())
    loc = (dev(qsl), dev(wl.seq_lens), cache, dev(wl.block_tables), max_q)
    for G in (32, 64):
        o8 = K.prefix_prefill_int8(d, q8, torch.full_like(qs, 2.0 ** -6), *loc, w_group=G)
        ob = K.prefix_prefill_bf16qk(d, dev(qb.view(np.int16)), *loc, w_group=G)
        torch.cuda.synchronize()
        assert_bits_equal(ob.cpu().numpy(), o8.cpu().numpy(), f"D={D} G={G} bf16-QK vs int8")


def test_prefill_bf16qk_cfg4_every_row_tile(orc):
    """First and last row of each of the 64 row tiles of 32, all 24 heads."""
    wl = W.cfg4_prefill()
    run_prefill_bf16qk(wl, orc, rows=row_tile_ends(2048))
