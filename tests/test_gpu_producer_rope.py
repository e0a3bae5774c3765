"""GPU parity of the producer with the rotary embedding fused in: int8
caches, fp32 scales and the int8 query with its scale bit-identical to the
oracle's (rotate-half pairing, fp32 products and sums rounded separately)."""
import numpy as np
import pytest

import workloads as W
from gpu_helpers import assert_bits_equal, cache_to_np, dev, desc_of, say, split_tokens

pytestmark = pytest.mark.gpu


def gpu_fill_rope(wl, positions, cos_sin):
    import int8_kv_quantized_amd as K
    d = desc_of(wl)
    cache = K.PagedCache.allocate(d)
    cs = dev(cos_sin)
    hist, qi = split_tokens(wl)
    if hist.size:
        K.kv_quantize_write_rope(d, dev(wl.key[hist]), dev(wl.value[hist]),
                                 dev(wl.slot_mapping[hist]), dev(positions[hist]), cs, cache)
    q8, qs = K.kv_quantize_write_rope(d, dev(wl.key[qi]), dev(wl.value[qi]),
                                      dev(wl.slot_mapping[qi]), dev(positions[qi]), cs, cache,
                                      query=dev(wl.query))
    return d, cache, q8, qs


def orc_fill_rope(orc, wl, positions, cos_sin):
    cache = orc.empty_cache(wl.num_blocks, wl.num_kv_heads, wl.head_dim)
    hist, qi = split_tokens(wl)
    if hist.size:
        orc.kv_quantize_write_rope(wl.key[hist], wl.value[hist], wl.slot_mapping[hist],
                                   positions[hist], cos_sin, cache, num_q_heads=wl.num_q_heads)
    q8, qs = orc.kv_quantize_write_rope(wl.key[qi], wl.value[qi], wl.slot_mapping[qi],
                                        positions[qi], cos_sin, cache,
                                        num_q_heads=wl.num_q_heads, query=wl.query)
    return cache, q8, qs


def _compare(orc, wl, positions, cos_sin, oracle_positions=None):
    say(f"  rope producer case {wl.name}: T={wl.num_tokens} Hq={wl.num_q_heads} "
        f"Hkv={wl.num_kv_heads} D={wl.head_dim} R={cos_sin.shape[1]} P={cos_sin.shape[0]}")
    d, cache, q8, qs = gpu_fill_rope(wl, positions, cos_sin)
    opos = positions if oracle_positions is None else oracle_positions
    ocache, oq8, oqs = orc_fill_rope(orc, wl, opos, cos_sin)
    g = cache_to_np(cache)
    for k in ("k_cache", "v_cache", "k_scale", "v_scale"):
        assert_bits_equal(g[k], ocache[k], f"{wl.name} {k}")
    assert_bits_equal(q8.cpu().numpy(), oq8, f"{wl.name} q_int8")
    assert_bits_equal(qs.cpu().numpy(), oqs, f"{wl.name} q_scale")
    return d, cache, q8, qs, ocache, oq8, oqs


SMALL = [
    dict(name="d256_r256_g6", seq_lens=(33, 17), num_q_heads=24, num_kv_heads=4, head_dim=256,
         R=256),
    dict(name="d256_r64_g6", seq_lens=(40, 9), num_q_heads=24, num_kv_heads=4, head_dim=256,
         R=64),
    dict(name="d256_r8", seq_lens=(21,), num_q_heads=4, num_kv_heads=1, head_dim=256, R=8),
    dict(name="d128_r128_mha", seq_lens=(37, 70), num_q_heads=8, num_kv_heads=8, head_dim=128,
         R=128),
    dict(name="d128_r4", seq_lens=(19,), num_q_heads=6, num_kv_heads=2, head_dim=128, R=4),
    dict(name="d64_r64", seq_lens=(5, 70), num_q_heads=4, num_kv_heads=4, head_dim=64, R=64),
    dict(name="d64_r2", seq_lens=(16, 3), num_q_heads=4, num_kv_heads=2, head_dim=64, R=2),
]


@pytest.mark.parametrize("kw", SMALL, ids=lambda k: k["name"])
@pytest.mark.parametrize("table", ["standard", "random"])
def test_rope_producer_small(orc, kw, table):
    kw = dict(kw)
    name, R = kw.pop("name"), kw.pop("R")
    wl = W.make_workload(name, new_tokens=[min(3, L) for L in kw["seq_lens"]], seed=51, **kw)
    rng = np.random.default_rng(52)
    if table == "standard":
        cs = W.rope_cos_sin(int(wl.seq_lens.max()), R)
        pos = wl.token_pos
    else:
        cs = W.random_cos_sin(rng, 97, R)
        pos = rng.integers(0, 97, wl.num_tokens).astype(np.int32)
    _compare(orc, wl, pos, cs)


CHUNK = [
    dict(name="chunk_d256_r256", num_q_heads=24, num_kv_heads=4, head_dim=256, R=256),
    dict(name="chunk_d256_r64", num_q_heads=24, num_kv_heads=4, head_dim=256, R=64),
    dict(name="chunk_d128_r128", num_q_heads=8, num_kv_heads=2, head_dim=128, R=128),
    dict(name="chunk_d128_r4", num_q_heads=6, num_kv_heads=2, head_dim=128, R=4),
    dict(name="chunk_d64_r64", num_q_heads=4, num_kv_heads=4, head_dim=64, R=64),
    dict(name="chunk_d64_r2", num_q_heads=4, num_kv_heads=2, head_dim=64, R=2),
]


@pytest.mark.parametrize("kw", CHUNK, ids=lambda k: k["name"])
@pytest.mark.parametrize("table", ["standard", "random"])
def test_rope_producer_chunks(orc, kw, table):
    """Calls of 128 tokens or more (the 16-token-per-wave kernel, with the
    table rows prefetched when the rotation covers the whole head): both
    calls of the fill are chunks (221 history tokens, 203 new ones with
    their queries), 16-token groups straddle sequences and pages, the last
    group is ragged, and some slots are skipped."""
    kw = dict(kw)
    name, R = kw.pop("name"), kw.pop("R")
    wl = W.make_workload(name, seq_lens=(290, 134), new_tokens=(141, 62), seed=57, **kw)
    wl.slot_mapping[7::37] = -1
    rng = np.random.default_rng(58)
    if table == "standard":
        cs = W.rope_cos_sin(int(wl.seq_lens.max()), R)
        pos = wl.token_pos
    else:
        cs = W.random_cos_sin(rng, 301, R)
        pos = rng.integers(0, 301, wl.num_tokens).astype(np.int32)
    hist, qi = split_tokens(wl)
    assert hist.size >= 128 and qi.size >= 128
    _compare(orc, wl, pos, cs)


def test_rope_identity_table_matches_plain_producer(orc):
    """cos 1 / sin 0 everywhere: the same bits as the producer without RoPE."""
    from gpu_helpers import gpu_fill
    wl = W.make_workload("ident", seq_lens=[40, 7], new_tokens=[2, 2], num_q_heads=8,
                         num_kv_heads=2, head_dim=128, seed=53)
    R = 128
    ident = np.concatenate([np.ones((64, R // 2), np.float32),
                            np.zeros((64, R // 2), np.float32)], 1)
    say("  rope producer case identity table")
    _, cache, q8, qs = gpu_fill_rope(wl, wl.token_pos, ident)
    _, pcache, pq8, pqs = gpu_fill(wl)
    g, p = cache_to_np(cache), cache_to_np(pcache)
    for k in g:
        assert_bits_equal(g[k], p[k], f"identity {k}")
    assert_bits_equal(q8.cpu().numpy(), pq8.cpu().numpy(), "identity q_int8")
    assert_bits_equal(qs.cpu().numpy(), pqs.cpu().numpy(), "identity q_scale")


def test_rope_tiny_values_zeros_and_skipped_slots(orc):
    wl = W.make_workload("tiny_rope", seq_lens=[48], new_tokens=[4], num_q_heads=4,
                         num_kv_heads=2, head_dim=256, seed=54)
    rng = np.random.default_rng(54)
    wl.key[:8] = W.f32_to_bf16_bits((rng.standard_normal(wl.key[:8].shape) * 1e-38)
                                    .astype(np.float32))
    wl.key[8:12] = 0
    wl.value[12:16] = 0
    wl.slot_mapping[::5] = -1
    _compare(orc, wl, wl.token_pos, W.rope_cos_sin(48, 128))


def test_rope_out_of_range_positions_are_clamped(orc):
    """Documented device behaviour: a position outside the table reads the
    nearest row (here compared with the oracle given the clamped positions)."""
    wl = W.make_workload("clamp", seq_lens=[30], new_tokens=[3], num_q_heads=4, num_kv_heads=2,
                         head_dim=128, seed=55)
    P = 20
    cs = W.rope_cos_sin(P, 128)
    pos = wl.token_pos.copy()
    pos[0] = -7
    _compare(orc, wl, pos, cs, oracle_positions=np.clip(pos, 0, P - 1).astype(np.int32))


def test_rope_then_decode_matches_oracle(orc):
    """The rotated cache feeds the decode unchanged: decode output against the
    oracle's decode over the oracle's rotated cache."""
    import int8_kv_quantized_amd as K
    wl = W.small_case("rope_decode", seq_lens=(300, 37, 520), num_q_heads=24, num_kv_heads=4,
                      head_dim=256, seed=56)
    cs = W.rope_cos_sin(int(wl.seq_lens.max()), 256)
    d, cache, q8, qs, ocache, oq8, oqs = _compare(orc, wl, wl.token_pos, cs)
    out = K.paged_decode_int8(d, q8, qs, cache, dev(wl.block_tables), dev(wl.seq_lens),
                              wl.max_seq_len).cpu().numpy()
    ref = orc.paged_decode(oq8, oqs, ocache, wl.block_tables, wl.seq_lens,
                           num_q_heads=wl.num_q_heads)
    err = np.abs(out - ref)
    assert err.max() <= 1e-3 and err.mean() <= 1e-4, (err.max(), err.mean())


@pytest.mark.parametrize("builder", [lambda: W.cfg2_decode(16384), W.cfg4_prefill,
                                     W.cfg5_mha_producer_decode],
                         ids=["cfg2_16k", "cfg4", "cfg5"])
def test_rope_producer_full_configs(orc, builder):
    wl = builder()
    _compare(orc, wl, wl.token_pos, W.rope_cos_sin(int(wl.seq_lens.max()), wl.head_dim))
