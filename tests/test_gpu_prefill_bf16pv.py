"""GPU parity of the prefill BF16-PV ablation (W = p~ sV rounded to bf16
times the int8 V) against the oracle with ORC_BF16_PV and 64-key tiles (the
kernel's tile, whose running maximum the bf16 rounding depends on): max-abs
1e-3, mean-abs 1e-4.  The error of both PV variants against unquantized fp64
attention is reported."""
import numpy as np
import pytest

import workloads as W
from gpu_helpers import (assert_bits_equal, assert_close, cache_to_np, dev, gpu_fill,
                         oracle_rows, report_fp64, row_tile_ends, say)
from refmath import prefill_reference_fp64

pytestmark = pytest.mark.gpu


def run_prefill_bf16pv(wl, orc, rows=None):
    import torch

    import int8_kv_quantized_amd as K
    from oracle import ORC_BF16_PV
    say(f"  bf16-PV prefill case {wl.name}: S={wl.num_seqs} Tq={wl.query.shape[0]} "
        f"Lmax={wl.max_seq_len} Hq={wl.num_q_heads} Hkv={wl.num_kv_heads} D={wl.head_dim} "
        f"rows={'all' if rows is None else len(rows)}")
    d, cache, q8, qs = gpu_fill(wl)
    ocache, oq8, oqs = orc.fill(wl)
    g = cache_to_np(cache)
    for k in g:
        assert_bits_equal(g[k], ocache[k], f"{wl.name} {k}")
    qsl = wl.query_start_loc
    max_q = int((qsl[1:] - qsl[:-1]).max())
    args = (d, q8, qs, dev(qsl), dev(wl.seq_lens), cache, dev(wl.block_tables), max_q)
    out = K.prefix_prefill_bf16pv(*args)
    out8 = K.prefix_prefill_int8(*args, w_group=32)
    torch.cuda.synchronize()
    out, out8 = out.cpu().numpy(), out8.cpu().numpy()
    r = np.arange(out.shape[0], dtype=np.int32) if rows is None else np.asarray(rows, np.int32)
    ref = oracle_rows(lambda **kw: orc.prefix_prefill(oq8, oqs, qsl, wl.seq_lens, ocache,
                                                      wl.block_tables, tile=64,
                                                      flags=ORC_BF16_PV, **kw),
                      r, np.zeros_like(out))
    say(f"    compared {r.size} query rows x {wl.num_q_heads} heads")
    sel = r
    assert_close(out[sel], ref[sel], f"{wl.name} bf16-PV")
    ref64 = prefill_reference_fp64(wl, rows=r)
    report_fp64(out[sel], ref64[sel], f"{wl.name} bf16-PV")
    report_fp64(out8[sel], ref64[sel], f"{wl.name} int8-PV G=32")


SMALL = [
    dict(name="ragged_d128_g3", seq_lens=(40, 300, 33, 130, 700), new_tokens=(8, 50, 33, 1, 200),
         num_q_heads=6, num_kv_heads=2, head_dim=128),
    dict(name="d64_mha", seq_lens=(70, 129), new_tokens=(70, 64), num_q_heads=4, num_kv_heads=4,
         head_dim=64),
    dict(name="d256_g6", seq_lens=(600, 300), new_tokens=(100, 37), num_q_heads=24,
         num_kv_heads=4, head_dim=256),
]


@pytest.mark.parametrize("kw", SMALL, ids=lambda k: k["name"])
def test_prefill_bf16pv_small(orc, kw):
    kw = dict(kw)
    name = kw.pop("name")
    wl = W.make_workload(name, seed=91, kind="prefill", **kw)
    run_prefill_bf16pv(wl, orc)


def test_prefill_bf16pv_cfg4_every_row_tile(orc):
    """First and last row of each of the 64 row tiles of 32, all 24 heads."""
    wl = W.cfg4_prefill()
    run_prefill_bf16pv(wl, orc, rows=row_tile_ends(2048))
