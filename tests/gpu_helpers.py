"""Helpers for the GPU parity tests: move a workload to the device, run the
HIP path through the C ABI, and compare with the oracle."""
from __future__ import annotations

import sys

import numpy as np

import workloads as W


def say(*a):
    print(*a, file=sys.__stdout__, flush=True)


def dev(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def desc_of(wl):
    import int8_kv_quantized_amd as K
    return K.CacheDesc(wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.num_blocks)


def split_tokens(wl):
    is_q = np.zeros(wl.num_tokens, bool)
    is_q[wl.query_token_index] = True
    return np.nonzero(~is_q)[0], wl.query_token_index


def gpu_fill(wl):
    """Producer on the GPU: history tokens without Q, then the query tokens."""
    import int8_kv_quantized_amd as K
    d = desc_of(wl)
    cache = K.PagedCache.allocate(d)
    hist, qi = split_tokens(wl)
    if hist.size:
        K.kv_quantize_write(d, dev(wl.key[hist]), dev(wl.value[hist]),
                            dev(wl.slot_mapping[hist]), cache)
    q8, qs = K.kv_quantize_write(d, dev(wl.key[qi]), dev(wl.value[qi]),
                                 dev(wl.slot_mapping[qi]), cache, query=dev(wl.query))
    return d, cache, q8, qs


def cache_to_np(cache):
    return dict(k_cache=cache.k_cache.cpu().numpy(), v_cache=cache.v_cache.cpu().numpy(),
                k_scale=cache.k_scale.cpu().numpy(), v_scale=cache.v_scale.cpu().numpy())


def assert_bits_equal(a, b, what):
    a = np.ascontiguousarray(a)
    b = np.ascontiguousarray(b)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    if a.dtype.kind == "f":
        a, b = a.view(np.uint32), b.view(np.uint32)
    bad = np.count_nonzero(a != b)
    assert bad == 0, f"{what}: {bad} of {a.size} elements differ"


def assert_close(got, ref, what, max_abs=1e-3, mean_abs=1e-4):
    err = np.abs(got.astype(np.float64) - ref.astype(np.float64))
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    mx, mn = float(err.max()), float(err.mean())
    say(f"    {what}: max-abs {mx:.3e}  mean-abs {mn:.3e}")
    assert mx <= max_abs and mn <= mean_abs, f"{what}: max-abs {mx:.3e} mean-abs {mn:.3e}"
    return mx, mn


def decode_queries(q8, qs, wl):
    """Rows of the producer's Q that are the decode queries (newest token)."""
    rows = wl.decode_query_rows()
    return q8[rows].contiguous(), qs[rows].contiguous()


def report_fp64(got, ref64, what):
    err = np.abs(got.astype(np.float64) - ref64)
    say(f"    {what} vs unquantized fp64 attention: max-abs {err.max():.3e} "
        f"mean-abs {err.mean():.3e}")


def host_workers(cap=16):
    """Threads for oracle work on the host: the CPUs this process may use, at
    most ``cap`` (the GPU machine gives one GPU's job a 16-CPU share)."""
    import os
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(cap, n))


def oracle_rows(fn, rows, out, workers=None, chunk=4):
    """Fill ``out`` at ``rows`` with ``fn(rows=<int32 array>, out=out)`` run
    over chunks of rows on a thread pool.  The oracle is a ctypes library, so
    each call releases the GIL and the chunks run in parallel; each call
    writes only its own rows of ``out``."""
    from concurrent.futures import ThreadPoolExecutor
    rows = np.asarray(rows, np.int32)
    parts = [rows[i:i + chunk] for i in range(0, rows.size, chunk)]
    with ThreadPoolExecutor(workers or host_workers()) as ex:
        list(ex.map(lambda r: fn(rows=r, out=out), parts))
    return out


def row_tile_ends(total_rows, tile=32):
    """First and last query row of every ``tile``-row tile of a chunk."""
    starts = np.arange(0, total_rows, tile)
    return np.unique(np.concatenate([starts, np.minimum(starts + tile - 1, total_rows - 1)]))


def prefill_tie_allowance(orc, q8, qs, qsl, seq_lens, cache, block_tables, row, head, G,
                          flags=0, delta=1e-4):
    """Per output dim of one prefill (row, head): the most the kernel may
    differ from the oracle because of W codes that sit at a rounding tie
    ("Implementing INT8 PV MMAC on a gfx936 DCU", section 1: Wq = round(W / sW),
    with W = p~ sV of section 2.1).

    A code is decided by rounding W / sW; where that quotient lies within
    `delta` of a half-integer, the kernel's own fp32 W (base-2 exponential,
    its reference max, a reciprocal, ties to even) may fall on the other side
    of the tie than the oracle's IEEE quotient, and either code is a correct
    decision.  Changing one such code by one unit moves the output by
    sW |Vq[d]| / l; the allowance is the sum over the row's tie codes (zero
    for a row without one).  Codes: the oracle's trace of the row."""
    t = orc.prefill_row(q8, qs, qsl, seq_lens, cache, block_tables, row, head, w_group=G,
                        flags=flags)
    nk = t["nk"]
    keys = np.arange(nk)
    b = int(np.searchsorted(qsl, row, side="right") - 1)
    Hq = q8.shape[1]
    Hkv = cache["k_cache"].shape[1]
    kv = head // (Hq // Hkv)
    page = block_tables[b, keys // 16]
    off = keys % 16
    sv = cache["v_scale"][page, off, kv]
    vq = cache["v_cache"][page, kv, :, off].astype(np.float64)       # [nk, D]
    W = (t["ptil"] * sv).astype(np.float32)
    sW = t["sW"][keys // G].astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(sW > 0, W / np.where(sW > 0, sW, 1), 0).astype(np.float64)
    tie = (sW > 0) & (np.abs(q - np.floor(q) - 0.5) <= delta)
    return (sW[tie, None].astype(np.float64) * np.abs(vq[tie])).sum(axis=0) / float(t["l"][0])


def assert_close_prefill(got, ref, rows, tie_fn, what, max_abs=1e-3, mean_abs=1e-4):
    """assert_close for prefill rows, except that an element of a (row, head)
    whose max-abs exceeds max_abs may differ by max_abs plus that row's tie
    allowance (tie_fn(row, head) -> per-dim allowance; prefill_tie_allowance).
    mean-abs is checked over everything, unchanged."""
    err = np.abs(got.astype(np.float64) - ref.astype(np.float64))
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    mx, mn = float(err.max()), float(err.mean())
    say(f"    {what}: max-abs {mx:.3e}  mean-abs {mn:.3e}")
    assert mn <= mean_abs, f"{what}: mean-abs {mn:.3e}"
    over = np.argwhere(err.max(axis=2) > max_abs)
    for i, h in over:
        a = tie_fn(int(rows[i]), int(h))
        assert a.max() > 0, f"{what}: row {rows[i]} head {h} max-abs {err[i, h].max():.3e}, no tie code"
        assert np.all(err[i, h] <= max_abs + a), (
            f"{what}: row {rows[i]} head {h} max-abs {err[i, h].max():.3e} beyond its tie codes")
    if over.size:
        say(f"    {len(over)} (row, head) pairs past {max_abs:g}, each explained by W codes at a "
            f"rounding tie")
    return mx, mn
