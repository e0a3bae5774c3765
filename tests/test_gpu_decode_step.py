"""GPU tests of the fused decode step (i8kv_decode_step_int8).

The step must equal the producer followed by the decode, bit for bit: the
caches and scales it writes, the quantized queries it returns and the
attention output are compared with i8kv_kv_quantize_write +
i8kv_paged_decode_int8 run on a copy of the same cache, and the output is
also checked against the oracle (max-abs 1e-3, mean-abs 1e-4).
"""
import numpy as np
import pytest

import workloads as W
from gpu_helpers import (assert_bits_equal, assert_close, cache_to_np, desc_of, dev,
                         split_tokens, say)

pytestmark = pytest.mark.gpu


def run_step(wl, orc, G, zero_len=()):
    import int8_kv_quantized_amd as K
    import torch
    say(f"  decode step case {wl.name}: S={wl.num_seqs} Lmax={wl.max_seq_len} "
        f"Hq={wl.num_q_heads} Hkv={wl.num_kv_heads} D={wl.head_dim} G={G} zero_len={list(zero_len)}")
    d = desc_of(wl)
    hist, qi = split_tokens(wl)
    rows = wl.decode_query_rows()          # query row of each sequence (its newest token)
    newest = qi[rows]                      # token index of each sequence's newest token
    lens = wl.seq_lens.astype(np.int32).copy()
    for s in zero_len:
        lens[s] = 0
    base = K.PagedCache.allocate(d)
    if hist.size:
        K.kv_quantize_write(d, dev(wl.key[hist]), dev(wl.value[hist]), dev(wl.slot_mapping[hist]),
                            base)
    sep = K.PagedCache(base.k_cache.clone(), base.v_cache.clone(), base.k_scale.clone(),
                       base.v_scale.clone())
    bt, sl = dev(wl.block_tables), dev(lens)
    # producer + decode, the newest token only where the sequence is non-empty
    slots = wl.slot_mapping[newest].astype(np.int32).copy()
    slots[lens == 0] = -1
    q8, qs = K.kv_quantize_write(d, dev(wl.key[newest]), dev(wl.value[newest]), dev(slots), sep,
                                 query=dev(wl.query[rows]))
    out_sep = K.paged_decode_int8(d, q8, qs, sep, bt, sl, wl.max_seq_len, w_group=G)
    # fused step, twice on fresh copies: the result must not depend on the run
    outs = []
    for _ in range(2):
        fused = K.PagedCache(base.k_cache.clone(), base.v_cache.clone(), base.k_scale.clone(),
                             base.v_scale.clone())
        fq8 = torch.full_like(q8, 77)
        fqs = torch.full_like(qs, -1.0)
        out = K.decode_step_int8(d, dev(wl.key[newest]), dev(wl.value[newest]),
                                 dev(wl.query[rows]), fused, bt, sl, wl.max_seq_len, w_group=G,
                                 q_int8=fq8, q_scale=fqs)
        torch.cuda.synchronize()
        outs.append((out.cpu().numpy(), cache_to_np(fused), fq8.cpu().numpy(), fqs.cpu().numpy()))
    g_sep = cache_to_np(sep)
    o_sep = out_sep.cpu().numpy()
    for out, g, fq8, fqs in outs:
        for k in g:
            assert_bits_equal(g[k], g_sep[k], f"{wl.name} fused {k}")
        assert_bits_equal(fq8, q8.cpu().numpy(), f"{wl.name} fused q_int8")
        assert_bits_equal(fqs, qs.cpu().numpy(), f"{wl.name} fused q_scale")
        assert_bits_equal(out, o_sep, f"{wl.name} fused out")
    for s in zero_len:
        assert not outs[0][0][s].any()
    # and the oracle on the same (complete) cache
    ocache, oq8, oqs = orc.fill(wl)
    ref = orc.paged_decode(oq8[rows], oqs[rows], ocache, wl.block_tables, lens,
                           num_q_heads=wl.num_q_heads, w_group=G)
    live = np.array([s for s in range(wl.num_seqs) if s not in zero_len])
    assert_close(outs[0][0][live], ref[live], f"{wl.name} G={G} step")


CASES = [
    dict(name="step_ragged_d128_g3", seq_lens=(1, 16, 17, 255, 256, 257, 513, 700),
         num_q_heads=6, num_kv_heads=2, head_dim=128),
    dict(name="step_d64_g16", seq_lens=(40, 300, 1), num_q_heads=16, num_kv_heads=1, head_dim=64),
    dict(name="step_d256_g6", seq_lens=(600, 4097), num_q_heads=24, num_kv_heads=4, head_dim=256),
    dict(name="step_mha_d128", seq_lens=(1000, 16), num_q_heads=8, num_kv_heads=8, head_dim=128),
    # 122 partitions x 4 KV heads x 5 sequences: a grid of several rounds with
    # 6 KB of partials per workgroup (the non-temporal-store instantiations)
    dict(name="step_d256_g6_rounds", seq_lens=(20000, 1, 9000, 31000, 257), num_q_heads=24,
         num_kv_heads=4, head_dim=256),
    # 9 partitions x 2 KV heads x 40 sequences of seeded lengths: several rounds
    # with 1 KB of partials per workgroup (the several-rounds instantiation
    # without the non-temporal stores); most workgroups lie past their sequence
    dict(name="step_d128_g2_rounds",
         seq_lens=tuple(int(x) for x in np.random.default_rng(74).integers(1, 2200, 40)),
         num_q_heads=4, num_kv_heads=2, head_dim=128),
    # 16 q heads per KV head at D = 256 over 30 sequences of seeded lengths:
    # several rounds with the largest staged partials (16 rows x 256 dims)
    # and the fused quantization of 16 queries per workgroup
    dict(name="step_d256_g16_rounds",
         seq_lens=tuple(int(x) for x in np.random.default_rng(75).integers(1, 4000, 30)),
         num_q_heads=16, num_kv_heads=1, head_dim=256),
]


@pytest.mark.parametrize("G", [32, 64])
@pytest.mark.parametrize("kw", CASES, ids=lambda k: k["name"])
def test_decode_step_matches_producer_then_decode(orc, kw, G):
    kw = dict(kw)
    name = kw.pop("name")
    wl = W.make_workload(name, new_tokens=[1] * len(kw["seq_lens"]), seed=71, w_group=G, **kw)
    run_step(wl, orc, G)


def test_decode_step_empty_sequence(orc):
    wl = W.make_workload("step_empty", seq_lens=(300, 20, 257), new_tokens=[1, 1, 1],
                         num_q_heads=6, num_kv_heads=2, head_dim=128, seed=72)
    run_step(wl, orc, 32, zero_len=(1,))


@pytest.mark.parametrize("G", [32, 64])
def test_decode_step_cfg2_16k(orc, G):
    run_step(W.cfg2_decode(16384, G), orc, G)
