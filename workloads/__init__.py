"""Seeded synthetic inputs for paged attention over an int8 KV cache.

This module only draws random numbers and lays them out: bf16 bit patterns
for Q/K/V, block tables, slot mappings and sequence lengths.  It holds none
of the method's arithmetic (no quantization, no attention), so both the CPU
oracle and the HIP path can consume exactly the same inputs.

Every workload follows the shapes of the pages' decode / prefill studies
(24 query heads, 4 KV heads, head_dim 256, page size 16; the MHA producer case
uses 32 heads of dim 128).  Values are drawn as float32 and rounded to bf16
(round-to-nearest-even).  Sub-streams come from
``numpy.random.SeedSequence(seed).spawn`` so that each quantity has its own
independent generator.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional

import numpy as np

BLOCK_SIZE = 16


# --------------------------------------------------------------------------
# bf16 bit patterns
# --------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounding = ((u >> 16) & 1) + 0x7FFF
    out = ((u + rounding) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------
# Paging
# --------------------------------------------------------------------------
def deal_block_tables(rng: np.random.Generator, capacities: List[int],
                      block_size: int = BLOCK_SIZE, spare_blocks: int = 0):
    """Deal a randomly permuted pool of physical pages to sequences in order.

    ``capacities[s]`` is the number of token slots sequence ``s`` needs.
    Returns ``(block_tables [S, max_blocks] int32, num_blocks)``; unused table
    entries are 0 (a valid page id, never read for positions >= capacity).
    """
    nblk = [int(math.ceil(c / block_size)) for c in capacities]
    pool = int(sum(nblk)) + spare_blocks
    perm = rng.permutation(pool).astype(np.int32)
    max_blocks = max(1, max(nblk) if nblk else 1)
    tables = np.zeros((len(capacities), max_blocks), dtype=np.int32)
    pos = 0
    for s, n in enumerate(nblk):
        tables[s, :n] = perm[pos:pos + n]
        pos += n
    return tables, pool


def slots_for(tables: np.ndarray, seq: int, positions: np.ndarray,
              block_size: int = BLOCK_SIZE) -> np.ndarray:
    """Physical slot (page * block_size + offset) of each token position."""
    positions = np.asarray(positions, dtype=np.int64)
    pages = tables[seq, positions // block_size].astype(np.int64)
    return (pages * block_size + positions % block_size).astype(np.int32)


# --------------------------------------------------------------------------
# Workload description
# --------------------------------------------------------------------------
@dataclasses.dataclass
class Workload:
    """A fully materialized synthetic case.

    Cache tokens are listed sequence by sequence; ``key``/``value`` hold the
    bf16 bits of every token that ends up in the cache, ``slot_mapping`` the
    slot each of them is written to.  ``query`` holds bf16 bits for the tokens
    that also produce an int8 query (``query_token_index`` indexes ``key``).
    """
    name: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    seq_lens: np.ndarray            # [S] int32, cache length after the step
    block_tables: np.ndarray        # [S, max_blocks] int32
    key: np.ndarray                 # [T, Hkv, D] uint16 (bf16 bits)
    value: np.ndarray               # [T, Hkv, D] uint16
    slot_mapping: np.ndarray        # [T] int32
    token_seq: np.ndarray           # [T] int32   sequence of each cache token
    token_pos: np.ndarray           # [T] int32   position of each cache token
    query: np.ndarray               # [Tq, Hq, D] uint16
    query_token_index: np.ndarray   # [Tq] int64 index into key/value rows
    query_start_loc: np.ndarray     # [S+1] int32 (prefill: chunk rows per seq)
    kind: str                       # "decode" | "prefill"
    seed: int
    w_group: int = 32
    partition_size: int = 256
    note: str = ""

    @property
    def num_seqs(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def num_tokens(self) -> int:
        return int(self.key.shape[0])

    @property
    def softmax_scale(self) -> float:
        return float(np.float32(1.0 / math.sqrt(self.head_dim)))

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max()) if self.num_seqs else 0

    def effective_kv_bytes(self) -> int:
        """K + V int8 plus two fp32 scales per (token, KV head) read by decode."""
        per_tok = self.num_kv_heads * (2 * self.head_dim + 8)
        return int(self.seq_lens.astype(np.int64).sum()) * per_tok

    def decode_query_rows(self) -> np.ndarray:
        """Row of ``query`` that is each sequence's decode query (its newest)."""
        return (self.query_start_loc[1:] - 1).astype(np.int64)


def _streams(seed: int, n: int) -> List[np.random.Generator]:
    return [np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(n)]


def _normal_bf16(rng: np.random.Generator, shape) -> np.ndarray:
    return f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32))


def make_workload(name: str, *, seq_lens, new_tokens, num_q_heads: int,
                  num_kv_heads: int, head_dim: int, seed: int,
                  kind: str = "decode", v_outlier_frac: float = 0.0,
                  v_outlier_gain: float = 20.0, k_channel_sigma: float = 0.0,
                  v_laplace: bool = False, w_group: int = 32,
                  block_size: int = BLOCK_SIZE, note: str = "") -> Workload:
    """Build a workload.

    ``seq_lens[s]`` is the cache length after the step; ``new_tokens[s]`` of
    those (the newest) are the tokens whose Q is also produced.  For decode the
    query of a sequence is its newest token; for prefill every new token is a
    query row (causal within the chunk).
    """
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    new_tokens = np.asarray(new_tokens, dtype=np.int32)
    S = seq_lens.shape[0]
    assert new_tokens.shape[0] == S and np.all(new_tokens <= seq_lens)
    g_table, g_q, g_k, g_v, g_out, g_chan = _streams(seed, 6)
    tables, num_blocks = deal_block_tables(g_table, [int(x) for x in seq_lens],
                                           block_size)
    T = int(seq_lens.astype(np.int64).sum())
    Hkv, Hq, D = num_kv_heads, num_q_heads, head_dim

    key_f = g_k.standard_normal((T, Hkv, D), dtype=np.float32)
    if k_channel_sigma > 0:
        offs = g_chan.standard_normal((Hkv, D), dtype=np.float32) * np.float32(k_channel_sigma)
        key_f += offs[None]
    if v_laplace:
        val_f = g_v.laplace(0.0, 1.0, size=(T, Hkv, D)).astype(np.float32)
    else:
        val_f = g_v.standard_normal((T, Hkv, D), dtype=np.float32)
    if v_outlier_frac > 0:
        n_out = max(1, int(round(v_outlier_frac * Hkv * D)))
        chans = g_out.choice(Hkv * D, size=n_out, replace=False)
        hh, dd = np.divmod(chans, D)
        val_f[:, hh, dd] *= np.float32(v_outlier_gain)
    key = f32_to_bf16_bits(key_f)
    del key_f
    value = f32_to_bf16_bits(val_f)
    del val_f

    token_seq = np.repeat(np.arange(S, dtype=np.int32), seq_lens)
    starts = np.concatenate([[0], np.cumsum(seq_lens.astype(np.int64))])
    token_pos = (np.arange(T, dtype=np.int64) - np.repeat(starts[:-1], seq_lens)).astype(np.int32)
    slot = np.empty(T, dtype=np.int32)
    for s in range(S):
        slot[starts[s]:starts[s + 1]] = slots_for(tables, s, np.arange(seq_lens[s]), block_size)

    q_idx = np.concatenate([np.arange(starts[s + 1] - new_tokens[s], starts[s + 1])
                            for s in range(S)]).astype(np.int64)
    query = _normal_bf16(g_q, (q_idx.shape[0], Hq, D))
    qsl = np.concatenate([[0], np.cumsum(new_tokens)]).astype(np.int32)
    return Workload(name=name, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                    block_size=block_size, num_blocks=num_blocks, seq_lens=seq_lens,
                    block_tables=tables, key=key, value=value, slot_mapping=slot,
                    token_seq=token_seq, token_pos=token_pos, query=query,
                    query_token_index=q_idx, query_start_loc=qsl, kind=kind,
                    seed=seed, w_group=w_group, note=note)


# --------------------------------------------------------------------------
# The five studied configurations (seed = 1000 + configuration number)
# --------------------------------------------------------------------------
GQA = dict(num_q_heads=24, num_kv_heads=4, head_dim=256)
MHA = dict(num_q_heads=32, num_kv_heads=32, head_dim=128)


def cfg1_decode_512(w_group: int = 32) -> Workload:
    """Decode, 1 seq, history 512, N(0,1) Q/K/V, permuted block table."""
    return make_workload("decode_L512", seq_lens=[512], new_tokens=[1], seed=1001,
                         w_group=w_group, **GQA)


def cfg2_decode(L: int, w_group: int = 32) -> Workload:
    """Decode, batch 1 at history L (4096/8192/16384); 1% of V channels x20."""
    return make_workload(f"decode_L{L}_outlierV_G{w_group}", seq_lens=[L], new_tokens=[1],
                         seed=1002, v_outlier_frac=0.01, w_group=w_group, **GQA)


def cfg3_decode_32k(w_group: int = 32) -> Workload:
    """Decode, batch 1 at history 32768, N(0,1)."""
    return make_workload("decode_L32768", seq_lens=[32768], new_tokens=[1], seed=1003,
                         w_group=w_group, **GQA)


def cfg3_decode_batch16(w_group: int = 32, lo: int = 1024, hi: int = 32768) -> Workload:
    """Decode, batch 16 with lengths uniform in [lo, hi] (seeded)."""
    rng = _streams(1003, 7)[6]
    lens = rng.integers(lo, hi + 1, size=16).astype(np.int32)
    return make_workload("decode_batch16_L1K-32K", seq_lens=lens, new_tokens=[1] * 16,
                         seed=1003 + 100, w_group=w_group, **GQA)


def cfg4_prefill(chunk: int = 2048, history: int = 16384, w_group: int = 32) -> Workload:
    """Chunked prefill: ``chunk`` causal queries over ``history`` cached tokens."""
    return make_workload(f"prefill_{chunk}_over_{history}_G{w_group}",
                         seq_lens=[history + chunk], new_tokens=[chunk], seed=1004,
                         kind="prefill", w_group=w_group, **GQA)


def cfg5_mha_producer_decode(w_group: int = 32, batch: int = 8, new: int = 8,
                             lo: int = 1024, hi: int = 16384) -> Workload:
    """MHA 32x128: 8 new tokens per seq written by the producer, then decode.

    K ~ N(0,1) + a fixed per-channel offset ~ N(0, sigma=2); V ~ Laplace(0,1).
    History lengths are uniform in [lo, hi]; the cache holds history + 8.
    """
    rng = _streams(1005, 7)[6]
    hist = rng.integers(lo, hi + 1, size=batch).astype(np.int32)
    return make_workload("mha_producer_decode_b8", seq_lens=hist + new,
                         new_tokens=[new] * batch, seed=1005, k_channel_sigma=2.0,
                         v_laplace=True, w_group=w_group, **MHA)


def producer_chunk(tokens: int, w_group: int = 32) -> Workload:
    """A prefill chunk of `tokens` new tokens of one sequence, every one with
    its query (the producer's chunk shapes: 2242 and 4096 tokens)."""
    return make_workload(f"producer_chunk_T{tokens}", seq_lens=[tokens], new_tokens=[tokens],
                         seed=1100 + tokens % 1000, kind="prefill", w_group=w_group, **GQA)


def small_case(name: str = "small", *, seq_lens=(37, 300, 16, 1), new_tokens=None,
               num_q_heads: int = 6, num_kv_heads: int = 2, head_dim: int = 128,
               seed: int = 7, kind: str = "decode", w_group: int = 32,
               **kw) -> Workload:
    """Small ragged case for fast parity tests (several pages, ragged tails)."""
    seq_lens = list(seq_lens)
    if new_tokens is None:
        new_tokens = [1] * len(seq_lens)
    return make_workload(name, seq_lens=seq_lens, new_tokens=new_tokens,
                         num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
                         head_dim=head_dim, seed=seed, kind=kind, w_group=w_group, **kw)


CONFIG_BUILDERS: Dict[str, object] = {
    "decode_L512": cfg1_decode_512,
    "decode_L4096": lambda G=32: cfg2_decode(4096, G),
    "decode_L8192": lambda G=32: cfg2_decode(8192, G),
    "decode_L16384": lambda G=32: cfg2_decode(16384, G),
    "decode_L32768": cfg3_decode_32k,
    "decode_batch16": cfg3_decode_batch16,
    "prefill_2048_over_16384": lambda G=32: cfg4_prefill(w_group=G),
    "mha_producer_decode": cfg5_mha_producer_decode,
}


# --------------------------------------------------------------------------
# Rotary tables (an input of the producer, like the activations)
# --------------------------------------------------------------------------
def rope_cos_sin(max_position: int, rotary_dim: int, base: float = 10000.0) -> np.ndarray:
    """The usual rotary table: angle(p, j) = p * base^(-2j/R) for j < R/2.

    Returns fp32 ``[max_position, R]``: cosines in the first R/2 columns,
    sines in the last R/2, each computed in fp64 and rounded once.
    """
    assert rotary_dim % 2 == 0 and rotary_dim >= 2
    h = rotary_dim // 2
    inv_freq = base ** (-2.0 * np.arange(h, dtype=np.float64) / rotary_dim)
    ang = np.arange(max_position, dtype=np.float64)[:, None] * inv_freq[None, :]
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)


def random_cos_sin(rng: np.random.Generator, max_position: int,
                   rotary_dim: int) -> np.ndarray:
    """A table of uniformly random angles (every quadrant), same layout."""
    h = rotary_dim // 2
    ang = rng.uniform(-np.pi, np.pi, (max_position, h))
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)
