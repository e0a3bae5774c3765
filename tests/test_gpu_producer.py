"""GPU parity of the fused producer: int8 caches, fp32 scales and the int8
query with its scale must be bit-identical to the oracle's."""
import numpy as np
import pytest

import workloads as W
from gpu_helpers import assert_bits_equal, cache_to_np, dev, desc_of, gpu_fill, say

pytestmark = pytest.mark.gpu


def _compare(wl, orc):
    say(f"  producer case {wl.name}: T={wl.num_tokens} Hq={wl.num_q_heads} "
        f"Hkv={wl.num_kv_heads} D={wl.head_dim}")
    d, cache, q8, qs = gpu_fill(wl)
    ocache, oq8, oqs = orc.fill(wl)
    g = cache_to_np(cache)
    for k in ("k_cache", "v_cache", "k_scale", "v_scale"):
        assert_bits_equal(g[k], ocache[k], f"{wl.name} {k}")
    assert_bits_equal(q8.cpu().numpy(), oq8, f"{wl.name} q_int8")
    assert_bits_equal(qs.cpu().numpy(), oqs, f"{wl.name} q_scale")


SMALL = [
    dict(name="ragged_d128_g3", seq_lens=(37, 300, 16, 1), num_q_heads=6, num_kv_heads=2,
         head_dim=128),
    dict(name="d64_mha", seq_lens=(5, 70), num_q_heads=4, num_kv_heads=4, head_dim=64),
    dict(name="d256_g6", seq_lens=(33, 17), num_q_heads=24, num_kv_heads=4, head_dim=256),
    dict(name="d256_g16", seq_lens=(40,), num_q_heads=16, num_kv_heads=1, head_dim=256),
]


@pytest.mark.parametrize("kw", SMALL, ids=lambda k: k["name"])
def test_producer_small(orc, kw):
    kw = dict(kw)
    name = kw.pop("name")
    wl = W.make_workload(name, new_tokens=[min(3, L) for L in kw["seq_lens"]], seed=41, **kw)
    _compare(wl, orc)


def test_producer_tiny_values_and_zeros(orc):
    """Subnormal scales, all-zero vectors and exact .5 ties."""
    wl = W.make_workload("tiny", seq_lens=[40], new_tokens=[4], num_q_heads=4, num_kv_heads=2,
                         head_dim=128, seed=42)
    rng = np.random.default_rng(42)
    tiny = (rng.standard_normal(wl.key.shape) * 1e-38).astype(np.float32)
    wl.key[:] = W.f32_to_bf16_bits(tiny)
    wl.value[:8] = 0
    ties = (rng.integers(-126, 127, wl.value[8:16].shape) + 0.5).astype(np.float32)
    ties[..., 0] = 127.0
    wl.value[8:16] = W.f32_to_bf16_bits(ties * np.float32(2.0 ** -3))
    _compare(wl, orc)


def test_producer_skips_negative_slots(orc):
    import int8_kv_quantized_amd as K
    wl = W.make_workload("skip", seq_lens=[50], new_tokens=[50], num_q_heads=4, num_kv_heads=2,
                         head_dim=128, seed=43)
    slots = wl.slot_mapping.copy()
    slots[::7] = -1
    say("  producer case skip: negative slots")
    d = desc_of(wl)
    cache = K.PagedCache.allocate(d)
    q8, qs = K.kv_quantize_write(d, dev(wl.key), dev(wl.value), dev(slots), cache,
                                 query=dev(wl.query))
    ocache = orc.empty_cache(wl.num_blocks, 2, 128)
    oq8, oqs = orc.kv_quantize_write(wl.key, wl.value, slots, ocache, num_q_heads=4,
                                     query=wl.query)
    g = cache_to_np(cache)
    for k in g:
        assert_bits_equal(g[k], ocache[k], f"skip {k}")
    assert_bits_equal(q8.cpu().numpy(), oq8, "skip q_int8")


@pytest.mark.parametrize("builder", [
    W.cfg1_decode_512, lambda: W.cfg2_decode(16384), W.cfg3_decode_32k,
    W.cfg3_decode_batch16, W.cfg4_prefill, W.cfg5_mha_producer_decode],
    ids=["cfg1", "cfg2_16k", "cfg3_32k", "cfg3_batch16", "cfg4", "cfg5"])
def test_producer_full_configs(orc, builder):
    _compare(builder(), orc)


def _producer_case(orc, T, D, slot_kind, seed, Hq=8, Hkv=2, with_query=True):
    """Producer over T tokens with a chosen slot pattern, against the oracle."""
    import int8_kv_quantized_amd as K
    rng = np.random.default_rng(seed)
    nb = (T + 15) // 16 + 3
    key = W.f32_to_bf16_bits(rng.standard_normal((T, Hkv, D), dtype=np.float32))
    value = W.f32_to_bf16_bits(rng.standard_normal((T, Hkv, D), dtype=np.float32))
    query = W.f32_to_bf16_bits(rng.standard_normal((T, Hq, D), dtype=np.float32))
    if slot_kind == "aligned":
        slots = np.arange(T, dtype=np.int32) + 16
    elif slot_kind == "offset5":
        slots = np.arange(T, dtype=np.int32) + 5
    elif slot_kind == "shuffled":
        slots = rng.permutation(nb * 16)[:T].astype(np.int32)
    else:  # aligned with holes: some tokens skip the write
        slots = np.arange(T, dtype=np.int32)
        slots[rng.choice(T, max(1, T // 9), replace=False)] = -1
    say(f"  producer path case T={T} D={D} slots={slot_kind}")
    d = K.CacheDesc(Hq, Hkv, D, nb)
    cache = K.PagedCache.allocate(d)
    q8, qs = K.kv_quantize_write(d, dev(key), dev(value), dev(slots), cache,
                                 query=dev(query) if with_query else None)
    ocache = orc.empty_cache(nb, Hkv, D)
    oq8, oqs = orc.kv_quantize_write(key, value, slots, ocache, num_q_heads=Hq,
                                     query=query if with_query else None)
    g = cache_to_np(cache)
    for k in g:
        assert_bits_equal(g[k], ocache[k], f"T={T} D={D} {slot_kind} {k}")
    if with_query:
        assert_bits_equal(q8.cpu().numpy(), oq8, f"T={T} D={D} {slot_kind} q_int8")
        assert_bits_equal(qs.cpu().numpy(), oqs, f"T={T} D={D} {slot_kind} q_scale")


@pytest.mark.parametrize("T", [1, 15, 64, 127, 128, 129, 300])
@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("slot_kind", ["aligned", "offset5", "shuffled", "holes"])
def test_producer_token_counts_and_slot_patterns(orc, T, D, slot_kind):
    """Both launch shapes (one vector per wave below 128 tokens, 16-token
    items above) and every store path: whole pages staged through LDS,
    unaligned or permuted slots token by token, skipped slots, ragged tails."""
    _producer_case(orc, T, D, slot_kind, seed=T * 7 + D)
