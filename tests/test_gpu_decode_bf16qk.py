"""GPU parity of the BF16-QK ablation of the decode (the bf16 query, not
quantized, against the int8 K codes on the bf16 matrix unit) against the
oracle's orc_paged_decode_bf16qk: max-abs 1e-3 and mean-abs 1e-4 (the dot
products differ from the oracle's fp64 sums only by fp32 accumulation order).
A bf16 query that is int8 codes times 2^-6 must reproduce the int8 path with
q_scale = 2^-6 bit for bit (its products and sums are then exact on both
units).  The error of both QK variants against unquantized fp64 attention is
reported."""
import numpy as np
import pytest

import workloads as W
from gpu_helpers import (assert_bits_equal, assert_close, cache_to_np, decode_queries, dev,
                         gpu_fill, report_fp64, say)
from refmath import decode_reference_fp64

pytestmark = pytest.mark.gpu


def run_bf16qk(wl, orc, G=32, report=True):
    import torch

    import int8_kv_quantized_amd as K
    say(f"  bf16-QK decode case {wl.name}: S={wl.num_seqs} Lmax={wl.max_seq_len} "
        f"Hq={wl.num_q_heads} Hkv={wl.num_kv_heads} D={wl.head_dim} G={G}")
    d, cache, q8, qs = gpu_fill(wl)
    ocache, oq8, oqs = orc.fill(wl)
    g = cache_to_np(cache)
    for k in g:
        assert_bits_equal(g[k], ocache[k], f"{wl.name} {k}")
    rows = wl.decode_query_rows()
    qb = np.ascontiguousarray(wl.query[rows])
    dqb = dev(qb.view(np.int16))
    bt, sl = dev(wl.block_tables), dev(wl.seq_lens)
    ws = torch.zeros(max(256, K.paged_decode_workspace_bytes(d, wl.num_seqs, wl.max_seq_len)),
                     dtype=torch.uint8, device="cuda")
    out = K.paged_decode_bf16qk(d, dqb, cache, bt, sl, wl.max_seq_len, w_group=G, workspace=ws)
    out2 = K.paged_decode_bf16qk(d, dqb, cache, bt, sl, wl.max_seq_len, w_group=G, workspace=ws)
    torch.cuda.synchronize()
    out, out2 = out.cpu().numpy(), out2.cpu().numpy()
    assert np.array_equal(out, out2), "repeated call differs"
    ref = orc.paged_decode_bf16qk(qb, ocache, wl.block_tables, wl.seq_lens, w_group=G)
    assert_close(out, ref, f"{wl.name} bf16-QK G={G}")
    if report:
        exact = decode_reference_fp64(wl)
        report_fp64(out, exact, f"{wl.name} bf16-QK G={G}")
        dq8, dqs = decode_queries(q8, qs, wl)
        out8 = K.paged_decode_int8(d, dq8, dqs, cache, bt, sl, wl.max_seq_len, w_group=G,
                                   workspace=ws)
        torch.cuda.synchronize()
        report_fp64(out8.cpu().numpy(), exact, f"{wl.name} int8-QK G={G}")
    return d, cache, bt, sl, ws, oq8[rows]


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
def test_bf16qk_small(orc, kw, G):
    kw = dict(kw)
    name = kw.pop("name")
    wl = W.make_workload(name, new_tokens=[1] * len(kw["seq_lens"]), seed=71, **kw)
    run_bf16qk(wl, orc, G=G, report=False)


@pytest.mark.parametrize("D", [64, 128, 256])
def test_bf16qk_power_of_two_query_matches_int8_path(orc, D):
    """q = int8 codes * 2^-6 in bf16 against the int8 path with q_scale = 2^-6:
    bit-identical outputs (exact products and sums on both matrix units)."""
    import torch

    import int8_kv_quantized_amd as K
    wl = W.make_workload(f"pow2_d{D}", seq_lens=[300, 1000, 17], new_tokens=[1, 1, 1],
                         num_q_heads=8, num_kv_heads=2, head_dim=D, seed=72)
    say(f"  bf16-QK power-of-two case D={D}")
    d, cache, q8, qs = gpu_fill(wl)
    dq8, dqs = decode_queries(q8, qs, wl)
    qb = W.f32_to_bf16_bits(dq8.cpu().numpy().astype(np.float32) * np.float32(2.0 ** -6))
    bt, sl = dev(wl.block_tables), dev(wl.seq_lens)
    for G in (32, 64):
        o8 = K.paged_decode_int8(d, dq8, torch.full_like(dqs, 2.0 ** -6), cache, bt, sl,
                                 wl.max_seq_len, w_group=G)
        ob = K.paged_decode_bf16qk(d, dev(qb.view(np.int16)), cache, bt, sl, wl.max_seq_len,
                                   w_group=G)
        torch.cuda.synchronize()
        assert_bits_equal(ob.cpu().numpy(), o8.cpu().numpy(), f"D={D} G={G} bf16-QK vs int8")


def test_bf16qk_outlier_channels(orc):
    wl = W.make_workload("outlier", seq_lens=[3000], new_tokens=[1], num_q_heads=24,
                         num_kv_heads=4, head_dim=256, seed=73, v_outlier_frac=0.01)
    run_bf16qk(wl, orc)


@pytest.mark.parametrize("L", [4096, 16384])
def test_bf16qk_full_configs(orc, L):
    run_bf16qk(W.cfg2_decode(L), orc)


def test_bf16qk_batch16_sampled(orc):
    """Batch 16, L ~ U[1K, 32K]: sampled sequences against the oracle."""
    import torch

    import int8_kv_quantized_amd as K
    wl = W.cfg3_decode_batch16()
    say(f"  bf16-QK decode batch16 sampled: S={wl.num_seqs} Lmax={wl.max_seq_len}")
    d, cache, q8, qs = gpu_fill(wl)
    rows = wl.decode_query_rows()
    qb = np.ascontiguousarray(wl.query[rows])
    out = K.paged_decode_bf16qk(d, dev(qb.view(np.int16)), cache, dev(wl.block_tables),
                                dev(wl.seq_lens), wl.max_seq_len)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    ocache = cache_to_np(cache)
    for b in (0, 7, 15):
        ref = orc.paged_decode_bf16qk(qb[b:b + 1], ocache, wl.block_tables[b:b + 1],
                                      wl.seq_lens[b:b + 1])
        assert_close(out[b:b + 1], ref, f"batch16 seq {b} bf16-QK")
