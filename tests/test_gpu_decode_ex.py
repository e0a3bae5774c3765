"""GPU parity of i8kv_paged_decode_ex: several causal queries per sequence
(each a one-query decode of the sequence cut after its position; K/V read
once), every PV variant, and bf16 output.

fp32 outputs: max-abs 1e-3, mean-abs 1e-4 against the oracle.  bf16 output:
bit-equal to the same call's fp32 output rounded to nearest-even (the kernel
rounds what it would have written), and within one bf16 ulp of |O| plus the
fp32 tolerance of the oracle's bf16-rounded output."""
import numpy as np
import pytest

import workloads as W
from gpu_helpers import assert_bits_equal, assert_close, cache_to_np, dev, gpu_fill, say

pytestmark = pytest.mark.gpu

PV_FLAG = {"int8": 0, "bf16": 4, "uint8": 8}


def multi_queries(q8, qs, wl, nq):
    """Rows s*nq + j: the nq newest query rows of each sequence (zeros where a
    sequence has fewer new tokens than nq)."""
    S, Hq, D = wl.num_seqs, wl.num_q_heads, wl.head_dim
    q8m = np.zeros((S * nq, Hq, D), np.int8)
    qsm = np.zeros((S * nq, Hq), np.float32)
    for b in range(S):
        rows = np.arange(wl.query_start_loc[b], wl.query_start_loc[b + 1])[-nq:]
        q8m[(b + 1) * nq - len(rows):(b + 1) * nq] = q8[rows]
        qsm[(b + 1) * nq - len(rows):(b + 1) * nq] = qs[rows]
    return q8m, qsm


def run_ex(orc, wl, nq, pv="int8", G=32, check_bf16=True):
    import torch

    import int8_kv_quantized_amd as K
    say(f"  decode_ex case {wl.name}: S={wl.num_seqs} Lmax={wl.max_seq_len} Hq={wl.num_q_heads} "
        f"Hkv={wl.num_kv_heads} D={wl.head_dim} nq={nq} pv={pv} G={G}")
    d, cache, q8, qs = gpu_fill(wl)
    ocache, oq8, oqs = orc.fill(wl)
    g = cache_to_np(cache)
    for k in g:
        assert_bits_equal(g[k], ocache[k], f"{wl.name} {k}")
    q8m, qsm = multi_queries(q8.cpu().numpy(), qs.cpu().numpy(), wl, nq)
    bt, sl = dev(wl.block_tables), dev(wl.seq_lens)
    out = K.paged_decode_ex(d, dev(q8m), dev(qsm), cache, bt, sl, wl.max_seq_len,
                            queries_per_seq=nq, pv=pv, w_group=G)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    ref = orc.paged_decode_multi(q8m, qsm, ocache, wl.block_tables, wl.seq_lens,
                                 num_q_heads=wl.num_q_heads, queries_per_seq=nq, w_group=G,
                                 flags=PV_FLAG[pv])
    assert_close(out, ref, f"{wl.name} nq={nq} pv={pv}")
    if check_bf16:
        ob = K.paged_decode_ex(d, dev(q8m), dev(qsm), cache, bt, sl, wl.max_seq_len,
                               queries_per_seq=nq, pv=pv, w_group=G, out_bf16=True)
        torch.cuda.synchronize()
        ob = ob.float().cpu().numpy()
        mine = torch.from_numpy(out).to(torch.bfloat16).float().numpy()
        assert_bits_equal(ob, mine, f"{wl.name} bf16 output vs own fp32 output rounded")
        refb = orc.round_bf16(ref)
        ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 1e-30))) - 7)
        assert np.all(np.abs(ob - refb) <= ulp + 1e-3), f"{wl.name} bf16 output vs oracle"
    return out, ref


CASES = [
    dict(name="gqa_d256_nq2", seq_lens=(33, 300, 520, 2), num_q_heads=24, num_kv_heads=4,
         head_dim=256, nq=2),
    dict(name="mha_d128_nq8", seq_lens=(257, 300, 700, 1000), num_q_heads=8, num_kv_heads=8,
         head_dim=128, nq=8),
    dict(name="d64_g2_nq8", seq_lens=(5, 264, 513), num_q_heads=4, num_kv_heads=2, head_dim=64,
         nq=8),
    dict(name="d128_g16_nq1", seq_lens=(40, 900), num_q_heads=16, num_kv_heads=1, head_dim=128,
         nq=1),
]


@pytest.mark.parametrize("pv", ["int8", "uint8", "bf16"])
@pytest.mark.parametrize("kw", CASES, ids=lambda k: k["name"])
def test_decode_ex(orc, kw, pv):
    kw = dict(kw)
    name, nq = kw.pop("name"), kw.pop("nq")
    wl = W.make_workload(name, new_tokens=[min(nq, L) for L in kw["seq_lens"]], seed=81, **kw)
    run_ex(orc, wl, nq, pv=pv, G=32, check_bf16=(pv == "int8"))


@pytest.mark.parametrize("G", [32, 64])
def test_decode_ex_mha_producer_config(orc, G):
    """The MHA configuration's 8 new tokens per sequence as 8 queries."""
    run_ex(orc, W.cfg5_mha_producer_decode(G), 8, G=G)


def test_decode_ex_nq1_equals_decode(orc):
    """nq = 1 with the int8 PV is the plain decode, bit for bit."""
    import torch

    import int8_kv_quantized_amd as K
    from gpu_helpers import decode_queries
    wl = W.make_workload("nq1", seq_lens=[300, 2000], new_tokens=[1, 1], num_q_heads=24,
                         num_kv_heads=4, head_dim=256, seed=82)
    say("  decode_ex case nq1 == decode")
    d, cache, q8, qs = gpu_fill(wl)
    dq8, dqs = decode_queries(q8, qs, wl)
    bt, sl = dev(wl.block_tables), dev(wl.seq_lens)
    a = K.paged_decode_ex(d, dq8, dqs, cache, bt, sl, wl.max_seq_len)
    b = K.paged_decode_int8(d, dq8, dqs, cache, bt, sl, wl.max_seq_len)
    torch.cuda.synchronize()
    assert_bits_equal(a.cpu().numpy(), b.cpu().numpy(), "nq=1 ex vs decode")
