"""GPU parity of the UINT8-W decode (W groups quantized to codes 0..255
against max W / 255; the kernel feeds Wq - 128 to the signed int8 MFMA and
adds 128 * the group's V column sums back) against the oracle with
ORC_UINT8_W: max-abs 1e-3 and mean-abs 1e-4.  The error of the int8 and
UINT8 variants against unquantized fp64 attention is reported."""
import numpy as np
import pytest

import workloads as W
from gpu_helpers import (assert_bits_equal, assert_close, cache_to_np, decode_queries, dev,
                         gpu_fill, report_fp64, say)
from refmath import decode_reference_fp64

pytestmark = pytest.mark.gpu


def run_uint8w(wl, orc, G, report=True):
    import torch

    import int8_kv_quantized_amd as K
    from oracle import ORC_UINT8_W
    say(f"  uint8-W decode case {wl.name}: S={wl.num_seqs} Lmax={wl.max_seq_len} "
        f"Hq={wl.num_q_heads} Hkv={wl.num_kv_heads} D={wl.head_dim} G={G}")
    d, cache, q8, qs = gpu_fill(wl)
    ocache, oq8, oqs = orc.fill(wl)
    g = cache_to_np(cache)
    for k in g:
        assert_bits_equal(g[k], ocache[k], f"{wl.name} {k}")
    dq8, dqs = decode_queries(q8, qs, wl)
    bt, sl = dev(wl.block_tables), dev(wl.seq_lens)
    ws = torch.zeros(max(256, K.paged_decode_workspace_bytes(d, wl.num_seqs, wl.max_seq_len)),
                     dtype=torch.uint8, device="cuda")
    out = K.paged_decode_uint8w(d, dq8, dqs, cache, bt, sl, wl.max_seq_len, w_group=G,
                                workspace=ws)
    out2 = K.paged_decode_uint8w(d, dq8, dqs, cache, bt, sl, wl.max_seq_len, w_group=G,
                                 workspace=ws)
    torch.cuda.synchronize()
    out, out2 = out.cpu().numpy(), out2.cpu().numpy()
    assert np.array_equal(out, out2), "repeated call differs"
    rows = wl.decode_query_rows()
    ref = orc.paged_decode(oq8[rows], oqs[rows], ocache, wl.block_tables, wl.seq_lens,
                           num_q_heads=wl.num_q_heads, w_group=G, flags=ORC_UINT8_W)
    assert_close(out, ref, f"{wl.name} uint8-W G={G}")
    if report:
        exact = decode_reference_fp64(wl)
        report_fp64(out, exact, f"{wl.name} uint8-W G={G}")
        out8 = K.paged_decode_int8(d, dq8, dqs, cache, bt, sl, wl.max_seq_len, w_group=G,
                                   workspace=ws)
        torch.cuda.synchronize()
        report_fp64(out8.cpu().numpy(), exact, f"{wl.name} int8-W G={G}")


SMALL = [
    dict(name="ragged_d128_g3", seq_lens=(37, 300, 16, 1, 700, 256, 257), num_q_heads=6,
         num_kv_heads=2, head_dim=128),
    dict(name="d64_mha", seq_lens=(5, 70, 513), num_q_heads=4, num_kv_heads=4, head_dim=64),
    dict(name="d256_g6", seq_lens=(33, 1024, 2000), num_q_heads=24, num_kv_heads=4,
         head_dim=256),
    dict(name="d256_g16", seq_lens=(40, 4000), num_q_heads=16, num_kv_heads=1, head_dim=256),
]


@pytest.mark.parametrize("G", [32, 64])
@pytest.mark.parametrize("kw", SMALL, ids=lambda k: k["name"])
def test_uint8w_small(orc, kw, G):
    kw = dict(kw)
    name = kw.pop("name")
    wl = W.make_workload(name, new_tokens=[1] * len(kw["seq_lens"]), seed=71, w_group=G, **kw)
    run_uint8w(wl, orc, G)


def test_uint8w_zero_values(orc):
    """All-zero V rows and keys: zero W groups (sW = 0) next to live ones."""
    wl = W.make_workload("zeros", seq_lens=[300, 64], new_tokens=[1, 1], num_q_heads=6,
                         num_kv_heads=2, head_dim=128, seed=72)
    wl.value[:40] = 0
    wl.key[100:140] = 0
    run_uint8w(wl, orc, 32, report=False)


@pytest.mark.parametrize("G", [32, 64])
def test_uint8w_full_config(orc, G):
    run_uint8w(W.cfg2_decode(16384, G), orc, G)
