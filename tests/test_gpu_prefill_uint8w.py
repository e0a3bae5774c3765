"""GPU parity of the UINT8-W prefill (W groups quantized to 0..255 against
max W / 255; the PV-MMAC page's section 6 candidate in the prefill's online
softmax) against the oracle with ORC_UINT8_W: max-abs 1e-3, mean-abs 1e-4.
Small ragged cases compare every output; the 2048-over-16384 chunk compares
the first and last row of each 32-row tile.  The error of the UINT8 and int8
W variants against unquantized fp64 attention is reported."""
import numpy as np
import pytest

import workloads as W
from gpu_helpers import (assert_bits_equal, assert_close, cache_to_np, dev, gpu_fill,
                         oracle_rows, report_fp64, row_tile_ends, say)
from refmath import prefill_reference_fp64

pytestmark = pytest.mark.gpu


def run_prefill_u8(wl, orc, G, rows=None):
    import torch

    import int8_kv_quantized_amd as K
    from oracle import ORC_UINT8_W
    say(f"  uint8-W prefill case {wl.name}: S={wl.num_seqs} Tq={wl.query.shape[0]} "
        f"Lmax={wl.max_seq_len} Hq={wl.num_q_heads} Hkv={wl.num_kv_heads} D={wl.head_dim} "
        f"G={G} rows={'all' if rows is None else len(rows)}")
    d, cache, q8, qs = gpu_fill(wl)
    ocache, oq8, oqs = orc.fill(wl)
    g = cache_to_np(cache)
    for k in g:
        assert_bits_equal(g[k], ocache[k], f"{wl.name} {k}")
    qsl = wl.query_start_loc
    max_q = int((qsl[1:] - qsl[:-1]).max())
    args = (d, q8, qs, dev(qsl), dev(wl.seq_lens), cache, dev(wl.block_tables), max_q)
    out = K.prefix_prefill_uint8w(*args, w_group=G)
    out8 = K.prefix_prefill_int8(*args, w_group=G)
    torch.cuda.synchronize()
    out, out8 = out.cpu().numpy(), out8.cpu().numpy()
    r = np.arange(out.shape[0], dtype=np.int32) if rows is None else np.asarray(rows, np.int32)
    ref = oracle_rows(lambda **kw: orc.prefix_prefill(oq8, oqs, qsl, wl.seq_lens, ocache,
                                                      wl.block_tables, w_group=G,
                                                      flags=ORC_UINT8_W, **kw),
                      r, np.zeros_like(out))
    say(f"    compared {r.size} query rows x {wl.num_q_heads} heads")
    assert_close(out[r], ref[r], f"{wl.name} uint8-W G={G}")
    ref64 = prefill_reference_fp64(wl, rows=r)
    report_fp64(out[r], ref64[r], f"{wl.name} uint8-W G={G}")
    report_fp64(out8[r], ref64[r], f"{wl.name} int8-W G={G}")


SMALL = [
    dict(name="ragged_d128_g3", seq_lens=(40, 300, 33, 130, 700), new_tokens=(8, 50, 33, 1, 200),
         num_q_heads=6, num_kv_heads=2, head_dim=128),
    dict(name="d64_mha", seq_lens=(70, 129), new_tokens=(70, 64), num_q_heads=4, num_kv_heads=4,
         head_dim=64),
    dict(name="d256_g6", seq_lens=(600, 300), new_tokens=(100, 37), num_q_heads=24,
         num_kv_heads=4, head_dim=256),
]


@pytest.mark.parametrize("G", [32, 64])
@pytest.mark.parametrize("kw", SMALL, ids=lambda k: k["name"])
def test_prefill_uint8w_small(orc, kw, G):
    kw = dict(kw)
    name = kw.pop("name")
    wl = W.make_workload(name, seed=121, kind="prefill", w_group=G, **kw)
    run_prefill_u8(wl, orc, G)


@pytest.mark.parametrize("G", [32, 64])
def test_prefill_uint8w_zero_values(orc, G):
    """All-zero value vectors (scale 0) and all-zero queries inside the chunk."""
    wl = W.make_workload("u8_zeros", seed=122, kind="prefill", w_group=G, seq_lens=(150, 90),
                         new_tokens=(70, 90), num_q_heads=6, num_kv_heads=2, head_dim=128)
    wl.value[3::5, 0, :] = 0
    wl.query[::7, :, :] = 0
    run_prefill_u8(wl, orc, G)


@pytest.mark.parametrize("G", [32, 64])
def test_prefill_uint8w_cfg4_every_row_tile(orc, G):
    run_prefill_u8(W.cfg4_prefill(w_group=G), orc, G, rows=row_tile_ends(2048))
