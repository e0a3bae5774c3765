"""Independent fp64 helpers used by the pins and parity reports.

* ``cache_rows`` re-derives the per-slot view of a paged cache with numpy
  reshapes/transposes (not with the oracle's index arithmetic), so it pins the
  cache layouts of the page "INT8 KV and INT8 MMAC attention inference
  optimisation on a gfx936 DCU", section 2.3:
  K [blocks, Hkv, D/16, block_size, 16], V [blocks, Hkv, D, block_size],
  scales [blocks, block_size, Hkv].
* ``attention_fp64`` is plain unquantized softmax attention in fp64 over the
  original bf16 values: the textbook definition that the quantized method
  approximates.
"""
from __future__ import annotations

import numpy as np

from workloads import bf16_bits_to_f32, slots_for


def cache_rows(cache):
    """Per-slot views: Kq, Vq [nb*bs, Hkv, D] int8; sK, sV [nb*bs, Hkv] fp32."""
    k, v = cache["k_cache"], cache["v_cache"]
    nb, H, D16, bs, x = k.shape
    assert x == 16
    D = D16 * 16
    K = k.transpose(0, 3, 1, 2, 4).reshape(nb * bs, H, D)
    V = v.transpose(0, 3, 1, 2).reshape(nb * bs, H, D)
    sK = cache["k_scale"].reshape(nb * bs, H)
    sV = cache["v_scale"].reshape(nb * bs, H)
    return K, V, sK, sV


def seq_slots(wl, seq, n=None):
    n = int(wl.seq_lens[seq]) if n is None else n
    return slots_for(wl.block_tables, seq, np.arange(n), wl.block_size)


def seq_tokens(wl, seq):
    """Rows of wl.key / wl.value that belong to ``seq``, in position order."""
    idx = np.nonzero(wl.token_seq == seq)[0]
    return idx[np.argsort(wl.token_pos[idx], kind="stable")]


def attention_fp64(q, k, v, scale):
    """softmax(q k^T * scale) v in fp64.  q [Nq, D], k/v [Nk, D]."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    s = (q @ k.T) * scale
    s -= s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    p /= p.sum(axis=-1, keepdims=True)
    return p @ v, p


def decode_reference_fp64(wl):
    """Unquantized fp64 decode attention over the bf16 inputs: [S, Hq, D]."""
    S, Hq, Hkv, D = wl.num_seqs, wl.num_q_heads, wl.num_kv_heads, wl.head_dim
    grp = Hq // Hkv
    out = np.zeros((S, Hq, D), np.float64)
    qrows = wl.decode_query_rows()
    scale = 1.0 / np.sqrt(D)
    for b in range(S):
        tok = seq_tokens(wl, b)
        K = bf16_bits_to_f32(wl.key[tok])
        V = bf16_bits_to_f32(wl.value[tok])
        Q = bf16_bits_to_f32(wl.query[qrows[b]])
        for h in range(Hq):
            o, _ = attention_fp64(Q[h][None], K[:, h // grp], V[:, h // grp], scale)
            out[b, h] = o[0]
    return out


def prefill_reference_fp64(wl, rows=None):
    """Unquantized causal fp64 attention for prefill query rows: [Tq, Hq, D]."""
    Hq, Hkv, D = wl.num_q_heads, wl.num_kv_heads, wl.head_dim
    grp = Hq // Hkv
    Tq = wl.query.shape[0]
    rows = np.arange(Tq) if rows is None else np.asarray(rows)
    out = np.zeros((Tq, Hq, D), np.float64)
    scale = 1.0 / np.sqrt(D)
    qsl = wl.query_start_loc
    for b in range(wl.num_seqs):
        tok = seq_tokens(wl, b)
        K = bf16_bits_to_f32(wl.key[tok])
        V = bf16_bits_to_f32(wl.value[tok])
        chunk = int(qsl[b + 1] - qsl[b])
        ctx = int(wl.seq_lens[b]) - chunk
        sel = rows[(rows >= qsl[b]) & (rows < qsl[b + 1])]
        for r in sel:
            pos = ctx + int(r - qsl[b])
            Q = bf16_bits_to_f32(wl.query[r])
            for h in range(Hq):
                o, _ = attention_fp64(Q[h][None], K[:pos + 1, h // grp],
                                      V[:pos + 1, h // grp], scale)
                out[r, h] = o[0]
    return out
