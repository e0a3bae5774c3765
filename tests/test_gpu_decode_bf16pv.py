"""GPU parity of the BF16-PV ablation of the decode (W = P*sV rounded to bf16
times the int8 V) against the oracle with ORC_BF16_PV: max-abs 1e-3 and
mean-abs 1e-4 (the only differences are fp32 accumulation orders).  The
error of both PV variants against unquantized fp64 attention is reported."""
import numpy as np
import pytest

import workloads as W
from gpu_helpers import (assert_bits_equal, assert_close, cache_to_np, decode_queries, dev,
                         gpu_fill, report_fp64, say)
from refmath import decode_reference_fp64

pytestmark = pytest.mark.gpu


def run_bf16pv(wl, orc, report=True):
    import torch

    import int8_kv_quantized_amd as K
    from oracle import ORC_BF16_PV
    say(f"  bf16-PV decode case {wl.name}: S={wl.num_seqs} Lmax={wl.max_seq_len} "
        f"Hq={wl.num_q_heads} Hkv={wl.num_kv_heads} D={wl.head_dim}")
    d, cache, q8, qs = gpu_fill(wl)
    ocache, oq8, oqs = orc.fill(wl)
    g = cache_to_np(cache)
    for k in g:
        assert_bits_equal(g[k], ocache[k], f"{wl.name} {k}")
    dq8, dqs = decode_queries(q8, qs, wl)
    bt, sl = dev(wl.block_tables), dev(wl.seq_lens)
    ws = torch.zeros(max(256, K.paged_decode_workspace_bytes(d, wl.num_seqs, wl.max_seq_len)),
                     dtype=torch.uint8, device="cuda")
    out = K.paged_decode_bf16pv(d, dq8, dqs, cache, bt, sl, wl.max_seq_len, workspace=ws)
    out2 = K.paged_decode_bf16pv(d, dq8, dqs, cache, bt, sl, wl.max_seq_len, workspace=ws)
    torch.cuda.synchronize()
    out, out2 = out.cpu().numpy(), out2.cpu().numpy()
    assert np.array_equal(out, out2), "repeated call differs"
    rows = wl.decode_query_rows()
    ref = orc.paged_decode(oq8[rows], oqs[rows], ocache, wl.block_tables, wl.seq_lens,
                           num_q_heads=wl.num_q_heads, flags=ORC_BF16_PV)
    assert_close(out, ref, f"{wl.name} bf16-PV")
    if report:
        exact = decode_reference_fp64(wl)
        report_fp64(out, exact, f"{wl.name} bf16-PV")
        out8 = K.paged_decode_int8(d, dq8, dqs, cache, bt, sl, wl.max_seq_len, w_group=32,
                                   workspace=ws)
        torch.cuda.synchronize()
        report_fp64(out8.cpu().numpy(), exact, f"{wl.name} int8-PV G=32")


SMALL = [
    dict(name="ragged_d128_g3", seq_lens=(37, 300, 16, 1, 700, 256, 257), num_q_heads=6,
         num_kv_heads=2, head_dim=128),
    dict(name="d64_mha", seq_lens=(5, 70, 513), num_q_heads=4, num_kv_heads=4, head_dim=64),
    dict(name="d256_g6", seq_lens=(33, 1024, 2000), num_q_heads=24, num_kv_heads=4,
         head_dim=256),
    dict(name="d256_g16", seq_lens=(40, 4000), num_q_heads=16, num_kv_heads=1, head_dim=256),
]


@pytest.mark.parametrize("kw", SMALL, ids=lambda k: k["name"])
def test_bf16pv_small(orc, kw):
    kw = dict(kw)
    name = kw.pop("name")
    wl = W.make_workload(name, new_tokens=[1] * len(kw["seq_lens"]), seed=61, **kw)
    run_bf16pv(wl, orc)


def test_bf16pv_outlier_channels(orc):
    """The pages' PV table workload shape: 1% of V channels x20."""
    wl = W.make_workload("outlier", seq_lens=[3000], new_tokens=[1], num_q_heads=24,
                         num_kv_heads=4, head_dim=256, seed=62, v_outlier_frac=0.01)
    run_bf16pv(wl, orc)


@pytest.mark.parametrize("L", [4096, 16384])
def test_bf16pv_full_configs(orc, L):
    run_bf16pv(W.cfg2_decode(L), orc)
