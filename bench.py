#!/usr/bin/env python3
"""Benchmark of the int8-KV paged-attention hot path on one MI355X.

A step is one pass of the hot path over one batch: the producer quantizes
and writes the new token's K/V (and its query) into the paged int8 cache and
paged decode attends over the whole history -- by default as the fused
decode_step_int8 call (one decode launch), with the two separate calls
(kv_quantize_write + paged_decode_int8) timed beside it.  The default
workload is decode at 16384 tokens of history (batch 1, 24 q / 4 KV heads,
head_dim 256, page 16, 1% of V channels x20, W group 32), with inputs
resident in HBM and rotated over enough distinct cache copies (>= 512 MB) to
defeat the 256 MB last-level cache.  The chunked-prefill path (2048 queries
over 16384 cached tokens) is timed as well and reported as int8 TOPS, and so
is the producer alone over 2242- and 4096-token chunks, with and without the
rotary embedding fused in, and the decode with its int8 PV against a bf16 PV
(the pages' PV comparison) at 4K, 8K and 16K tokens, and 8 causal queries per
sequence in one decode call on the MHA configuration.

Prints ONE JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
INT8_PEAK_TOPS = 5000.0      # MI355X dense int8 MFMA, TOP/s
METRIC = ("decode µs & effective KV GB/s (% HBM peak) at 16K; "
          "prefill-chunk int8 TOPS")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse_args():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="decode_L16384",
                   choices=["decode_L512", "decode_L4096", "decode_L8192", "decode_L16384",
                            "decode_L32768", "decode_batch16", "mha_producer_decode"])
    p.add_argument("--w-group", type=int, default=32, choices=[32, 64])
    p.add_argument("--min-rotation-mb", type=float, default=512.0)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-prefill", action="store_true")
    p.add_argument("--no-multi-query", action="store_true",
                   help="skip the 8-queries-per-sequence decode on the MHA configuration")
    p.add_argument("--no-pv-ablation", action="store_true",
                   help="skip the int8-PV vs bf16-PV decode comparison at 4K/8K/16K")
    p.add_argument("--no-producer-chunks", action="store_true",
                   help="skip the producer-alone timing over 2242- and 4096-token chunks")
    p.add_argument("--prefill-reps", type=int, default=10)
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    p.add_argument("--no-configs", action="store_true",
                   help="skip the per-configuration decode records (every configuration at "
                        "G=32 and 64)")
    p.add_argument("--config-steps", type=int, default=50)
    p.add_argument("--separate-step", action="store_true",
                   help="time the step as kv_quantize_write + paged_decode_int8 instead of "
                        "the fused decode_step_int8")
    p.add_argument("--no-graph", action="store_true",
                   help="launch eagerly instead of replaying HIP graphs (for counter runs)")
    p.add_argument("--copy-calibration-mb", type=float, default=0.0,
                   help="only run a plain device copy of this size (for scaling HBM "
                        "byte counters) and exit")
    return p.parse_args()


def build_workload(name, G):
    import workloads as W
    b = W.CONFIG_BUILDERS[name]
    return b(G)


def cache_bytes(d):
    nb, H, D = d.num_blocks, d.num_kv_heads, d.head_dim
    return nb * H * D * 16 * 2 + nb * 16 * H * 4 * 2


def time_decode(args, log_prefix=""):
    import numpy as np
    import torch

    import int8_kv_quantized_amd as K
    wl = build_workload(args.workload, args.w_group)
    d = K.CacheDesc(wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.num_blocks)
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    is_q = np.zeros(wl.num_tokens, bool)
    is_q[wl.query_token_index] = True
    hist = np.nonzero(~is_q)[0]
    qi = wl.query_token_index

    copies = max(1, math.ceil(args.min_rotation_mb * 1e6 / cache_bytes(d)))
    log(f"{log_prefix}workload {wl.name}: S={wl.num_seqs} L_max={wl.max_seq_len} "
        f"cache {cache_bytes(d) / 1e6:.1f} MB x {copies} copies")
    base = K.PagedCache.allocate(d)
    if hist.size:
        K.kv_quantize_write(d, dev(wl.key[hist]), dev(wl.value[hist]),
                            dev(wl.slot_mapping[hist]), base)
    caches = [base] + [K.PagedCache(base.k_cache.clone(), base.v_cache.clone(),
                                    base.k_scale.clone(), base.v_scale.clone())
                       for _ in range(copies - 1)]
    knew, vnew, snew, qnew = (dev(wl.key[qi]), dev(wl.value[qi]), dev(wl.slot_mapping[qi]),
                              dev(wl.query))
    T = int(qi.shape[0])
    q8 = torch.empty((T, d.num_q_heads, d.head_dim), dtype=torch.int8, device="cuda")
    qs = torch.empty((T, d.num_q_heads), dtype=torch.float32, device="cuda")
    per_seq = T // wl.num_seqs
    if per_seq == 1:
        dq8, dqs = q8, qs
    else:
        dq8 = torch.empty((wl.num_seqs, d.num_q_heads, d.head_dim), dtype=torch.int8,
                          device="cuda")
        dqs = torch.empty((wl.num_seqs, d.num_q_heads), dtype=torch.float32, device="cuda")
    bt, sl = dev(wl.block_tables), dev(wl.seq_lens)
    ws = torch.zeros(K.paged_decode_workspace_bytes(d, wl.num_seqs, wl.max_seq_len),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty((wl.num_seqs, d.num_q_heads, d.head_dim), dtype=torch.float32,
                      device="cuda")
    def producer(i):
        K.kv_quantize_write(d, knew, vnew, snew, caches[i % copies], query=qnew, q_int8=q8,
                            q_scale=qs)
        if per_seq != 1:
            dq8.copy_(q8.view(wl.num_seqs, per_seq, *q8.shape[1:])[:, -1])
            dqs.copy_(qs.view(wl.num_seqs, per_seq, -1)[:, -1])

    def decode(i):
        K.paged_decode_int8(d, dq8, dqs, caches[i % copies], bt, sl, wl.max_seq_len,
                            w_group=args.w_group, workspace=ws, out=out)

    def partials(i):  # the partition kernel alone (stage 1 of the decode call)
        K.paged_decode_partials(d, dq8, dqs, caches[i % copies], bt, sl, wl.max_seq_len,
                                w_group=args.w_group, workspace=ws)

    def step_separate(i):
        producer(i)
        decode(i)

    def step_fused(i):  # the same work as step_separate, in one decode launch
        K.decode_step_int8(d, knew, vnew, qnew, caches[i % copies], bt, sl, wl.max_seq_len,
                           w_group=args.w_group, workspace=ws, out=out, q_int8=q8, q_scale=qs)

    fused = per_seq == 1 and not args.separate_step
    step = step_fused if fused else step_separate

    # Launch-bound at these sizes: capture whole loops in HIP graphs so the
    # timed region is the GPU's work, not the Python launch rate.
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(3):
            step(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    def capture(fn, n):
        if args.no_graph:
            return lambda: [fn(i) for i in range(n)]
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(n):
                fn(i)
        return g.replay

    def replay_ms(g):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        g()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    g_warm = capture(step, max(args.warmup, 1))
    g_step = capture(step, args.steps)
    g_sep = capture(step_separate, args.steps) if fused else g_step
    g_dec = capture(decode, args.steps)
    g_part = capture(partials, args.steps)
    g_prod = capture(producer, args.steps)
    if args.warmup:
        replay_ms(g_warm)
    ms_total = replay_ms(g_step)
    sep_ms = replay_ms(g_sep) / args.steps if fused else ms_total / args.steps
    dec_ms = [replay_ms(g_dec) / args.steps for _ in range(5)]  # p50 over 5 batches
    part_ms = [replay_ms(g_part) / args.steps for _ in range(5)]
    prod_ms = [replay_ms(g_prod) / args.steps for _ in range(3)]
    decode(0)
    torch.cuda.synchronize()
    return dict(wl=wl, desc=d, copies=copies, ms_per_step=ms_total / args.steps, fused=fused,
                step_separate_us=1e3 * sep_ms,
                producer_us=1e3 * float(np.median(prod_ms)),
                decode_us=1e3 * float(np.median(dec_ms)), decode_us_runs=[1e3 * x for x in dec_ms],
                partition_us=1e3 * float(np.median(part_ms)),
                out=out.cpu().numpy())


def _graph_us(fn, steps, reps=3):
    """Median us per call of `steps` calls of fn(i) captured in one HIP graph."""
    import numpy as np
    import torch
    for i in range(2):
        fn(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(steps):
            fn(i)
    g.replay()
    runs = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        runs.append(1e3 * e0.elapsed_time(e1) / steps)
    return float(np.median(runs))


def measure_decode_config(wl, groups=(32, 64), steps=50, min_rotation_mb=512.0,
                          new_tokens_step=False):
    """One decode configuration at each W group: the decode call, its partition
    kernel alone (i8kv_paged_decode_partials) and, with ``new_tokens_step``,
    the producer of every sequence's new tokens (with Q) and producer + decode
    as one step.  Caches rotated over >= min_rotation_mb of copies.  Returns
    (record per G, GPU output per G for the accuracy check)."""
    import numpy as np
    import torch

    import int8_kv_quantized_amd as K
    d = K.CacheDesc(wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.num_blocks)
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    is_q = np.zeros(wl.num_tokens, bool)
    is_q[wl.query_token_index] = True
    hist = np.nonzero(~is_q)[0]
    qi = wl.query_token_index
    base = K.PagedCache.allocate(d)
    if hist.size:
        K.kv_quantize_write(d, dev(wl.key[hist]), dev(wl.value[hist]),
                            dev(wl.slot_mapping[hist]), base)
    knew, vnew, snew, qnew = (dev(wl.key[qi]), dev(wl.value[qi]), dev(wl.slot_mapping[qi]),
                              dev(wl.query))
    q8, qs = K.kv_quantize_write(d, knew, vnew, snew, base, query=qnew)
    rows = torch.from_numpy(wl.decode_query_rows()).cuda()
    dq8, dqs = q8[rows].contiguous(), qs[rows].contiguous()
    copies = max(1, math.ceil(min_rotation_mb * 1e6 / cache_bytes(d)))
    caches = [base] + [K.PagedCache(base.k_cache.clone(), base.v_cache.clone(),
                                    base.k_scale.clone(), base.v_scale.clone())
                       for _ in range(copies - 1)]
    bt, sl, L = dev(wl.block_tables), dev(wl.seq_lens), wl.max_seq_len
    ws = torch.empty(K.paged_decode_workspace_bytes(d, wl.num_seqs, L), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty((wl.num_seqs, d.num_q_heads, d.head_dim), dtype=torch.float32,
                      device="cuda")
    eff = wl.effective_kv_bytes()
    recs, outs = {}, {}
    for G in groups:
        decode = lambda i: K.paged_decode_int8(d, dq8, dqs, caches[i % copies], bt, sl, L,
                                               w_group=G, workspace=ws, out=out)
        part = lambda i: K.paged_decode_partials(d, dq8, dqs, caches[i % copies], bt, sl, L,
                                                 w_group=G, workspace=ws)
        us = _graph_us(decode, steps)
        pus = _graph_us(part, steps)
        r = dict(decode_us=round(us, 3), decode_gbs=round(eff / (us * 1e-6) / 1e9, 1),
                 decode_frac_hbm=round(eff / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                 partition_kernel_us=round(pus, 3),
                 partition_kernel_frac_hbm=round(eff / (pus * 1e-6) / 1e9 / HBM_PEAK_GBS, 4))
        if new_tokens_step:
            def producer(i):
                K.kv_quantize_write(d, knew, vnew, snew, caches[i % copies], query=qnew,
                                    q_int8=q8, q_scale=qs)

            def step(i):
                producer(i)
                dq8.copy_(q8[rows])
                dqs.copy_(qs[rows])
                decode(i)
            r["producer_us"] = round(_graph_us(producer, steps), 3)
            r["producer_tokens"] = int(qi.shape[0])
            r["step_us"] = round(_graph_us(step, steps), 3)
        decode(0)
        torch.cuda.synchronize()
        outs[G] = out.cpu().numpy()
        recs[f"G{G}"] = r
    del caches, base
    torch.cuda.empty_cache()
    return dict(workload=wl.name, effective_kv_bytes=eff, cache_copies_rotated=copies,
                batch=wl.num_seqs, max_seq_len=L, **recs), outs


def time_prefill(reps, G=32, graph=True, bf16pv=False, bf16qk=False, min_rotation_mb=512.0,
                 keep_rows=None, warm_s=0.25, uint8w=False):
    """The 2048-over-16384 prefill chunk; successive calls read distinct copies
    of the K/V cache (>= min_rotation_mb in all, as many as there are calls per
    timed batch) so the 256 MB last-level cache does not hold the K/V of the
    previous calls (10 calls x 38 MB between reuses at the defaults)."""
    import math

    import numpy as np
    import torch

    import int8_kv_quantized_amd as K
    import workloads as W
    wl = W.cfg4_prefill(w_group=G)
    d = K.CacheDesc(wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.num_blocks)
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    cache = K.PagedCache.allocate(d)
    is_q = np.zeros(wl.num_tokens, bool)
    is_q[wl.query_token_index] = True
    hist = np.nonzero(~is_q)[0]
    qi = wl.query_token_index
    K.kv_quantize_write(d, dev(wl.key[hist]), dev(wl.value[hist]), dev(wl.slot_mapping[hist]),
                        cache)
    q8, qs = K.kv_quantize_write(d, dev(wl.key[qi]), dev(wl.value[qi]),
                                 dev(wl.slot_mapping[qi]), cache, query=dev(wl.query))
    copies = max(1, math.ceil(min_rotation_mb * 1e6 / cache_bytes(d)))
    caches = [cache] + [K.PagedCache(cache.k_cache.clone(), cache.v_cache.clone(),
                                     cache.k_scale.clone(), cache.v_scale.clone())
                        for _ in range(copies - 1)]
    qsl, sl, bt = dev(wl.query_start_loc), dev(wl.seq_lens), dev(wl.block_tables)
    out = torch.empty((q8.shape[0], d.num_q_heads, d.head_dim), dtype=torch.float32,
                      device="cuda")
    chunk = int(qi.shape[0])
    if bf16pv:  # the BF16-PV ablation of the same call
        run = lambda i: K.prefix_prefill_bf16pv(d, q8, qs, qsl, sl, caches[i % copies], bt, chunk,
                                                out=out)
    elif uint8w:  # UINT8 W groups (codes 0..255 against max W / 255)
        run = lambda i: K.prefix_prefill_uint8w(d, q8, qs, qsl, sl, caches[i % copies], bt, chunk,
                                                w_group=G, out=out)
    elif bf16qk:  # the BF16-QK ablation: the bf16 queries instead of q8 / qs
        qb = dev(np.ascontiguousarray(wl.query).view(np.int16))
        run = lambda i: K.prefix_prefill_bf16qk(d, qb, qsl, sl, caches[i % copies], bt, chunk,
                                                w_group=G, out=out)
    else:
        run = lambda i: K.prefix_prefill_int8(d, q8, qs, qsl, sl, caches[i % copies], bt, chunk,
                                              w_group=G, out=out)
    for i in range(2):
        run(i)
    torch.cuda.synchronize()
    if graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(reps):
                run(i)
        replay = g.replay
    else:
        replay = lambda: [run(i) for i in range(reps)]
    # The chunk is compute-bound: over the first ~30 ms of sustained load its
    # calls speed up (about 1070 -> 880 us at G = 32, measured call by call),
    # so batches are timed only after `warm_s` seconds of back-to-back calls,
    # and the median of three batches is reported.
    t_end = time.perf_counter() + warm_s
    while time.perf_counter() < t_end:
        replay()
        torch.cuda.synchronize()
    runs = []
    for _ in range(3):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        replay()
        e1.record()
        torch.cuda.synchronize()
        runs.append(1e3 * e0.elapsed_time(e1) / reps)
    us = float(np.median(runs))
    hist_len = int(wl.seq_lens[0]) - chunk
    visible = sum(hist_len + j + 1 for j in range(chunk))  # causal pairs per head
    ops = 2 * 2 * d.head_dim * d.num_q_heads * visible
    rows_out = None
    if keep_rows is not None:  # the output rows kept for the accuracy check
        run(0)
        torch.cuda.synchronize()
        rows_out = out[torch.from_numpy(np.asarray(keep_rows)).cuda()].cpu().numpy()
    return dict(us=us, ops=ops, tops=ops / (us * 1e-6) / 1e12, workload=wl.name,
                cache_copies_rotated=copies, rows_out=rows_out, runs_us=[round(x, 1) for x in runs])


def time_producer_chunk(tokens, steps=50, min_rotation_mb=512.0):
    """The producer alone over a prefill chunk of `tokens` tokens (24 q / 4 KV
    heads, head_dim 256, every token with its query), without and with the
    rotary embedding fused in; inputs and caches rotated over enough copies
    to exceed the last-level cache.  Returns us per call and HBM GB/s of the
    algorithmic bytes (bf16 Q/K/V read, int8 codes and fp32 scales written,
    slot / position / table row read)."""
    import numpy as np
    import torch

    import int8_kv_quantized_amd as K
    import workloads as W
    wl = W.producer_chunk(tokens)
    d = K.CacheDesc(wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.num_blocks)
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    Hq, Hkv, D, T = wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.num_tokens
    R = D
    per_tok = 2 * (Hq + 2 * Hkv) * D + (Hq + 2 * Hkv) * D + 4 * (Hq + 2 * Hkv) + 4
    set_bytes = T * per_tok
    copies = max(1, math.ceil(min_rotation_mb * 1e6 / set_bytes))
    k0, v0, q0 = dev(wl.key), dev(wl.value), dev(wl.query)
    sets = [(k0, v0, q0)] + [(k0.clone(), v0.clone(), q0.clone()) for _ in range(copies - 1)]
    caches = [K.PagedCache.allocate(d) for _ in range(copies)]
    slot, pos = dev(wl.slot_mapping), dev(wl.token_pos)
    cs = dev(W.rope_cos_sin(T, R))
    q8 = [torch.empty((T, Hq, D), dtype=torch.int8, device="cuda") for _ in range(copies)]
    qs = [torch.empty((T, Hq), dtype=torch.float32, device="cuda") for _ in range(copies)]

    def plain(i):
        k, v, q = sets[i % copies]
        K.kv_quantize_write(d, k, v, slot, caches[i % copies], query=q, q_int8=q8[i % copies],
                            q_scale=qs[i % copies])

    def rope(i):
        k, v, q = sets[i % copies]
        K.kv_quantize_write_rope(d, k, v, slot, pos, cs, caches[i % copies], query=q,
                                 q_int8=q8[i % copies], q_scale=qs[i % copies])

    res = {}
    for name, fn, extra_b in (("plain", plain, 0), ("rope", rope, 4 + 4 * R)):
        us = _graph_us(fn, steps, reps=5)
        b = T * (per_tok + extra_b)
        res[f"{name}_us"] = round(us, 3)
        res[f"{name}_gbs"] = round(b / (us * 1e-6) / 1e9, 1)
    res["bytes_plain"] = T * per_tok
    return res


def time_pv_ablation(L, G=32, steps=50, min_rotation_mb=512.0):
    """The pages' PV comparison: the same decode call with the int8 PV (W
    group-quantized, int8 MFMA) and with a bf16 PV (W = P*sV in bf16, int8 V
    exact in bf16, bf16 MFMA), nothing else changed; a batch-1 decode at
    L tokens, 24 q / 4 KV heads x 256, 1% of V channels x20; the UINT8-W
    variant and the QK comparison (the bf16 query against the int8 K on the
    bf16 matrix unit) are timed beside them.  Returns us per call of each and
    the speed-ups of the int8 PV (bf16 PV us / int8 us) and of the int8 QK
    (bf16 QK us / int8 us)."""
    import numpy as np
    import torch

    import int8_kv_quantized_amd as K
    import workloads as W
    wl = W.cfg2_decode(L, G)
    d = K.CacheDesc(wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.num_blocks)
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    is_q = np.zeros(wl.num_tokens, bool)
    is_q[wl.query_token_index] = True
    hist = np.nonzero(~is_q)[0]
    qi = wl.query_token_index
    base = K.PagedCache.allocate(d)
    K.kv_quantize_write(d, dev(wl.key[hist]), dev(wl.value[hist]), dev(wl.slot_mapping[hist]), base)
    q8, qs = K.kv_quantize_write(d, dev(wl.key[qi]), dev(wl.value[qi]), dev(wl.slot_mapping[qi]),
                                 base, query=dev(wl.query))
    copies = max(1, math.ceil(min_rotation_mb * 1e6 / cache_bytes(d)))
    caches = [base] + [K.PagedCache(base.k_cache.clone(), base.v_cache.clone(),
                                    base.k_scale.clone(), base.v_scale.clone())
                       for _ in range(copies - 1)]
    bt, sl = dev(wl.block_tables), dev(wl.seq_lens)
    qb = dev(np.ascontiguousarray(wl.query[wl.decode_query_rows()]).view(np.int16))
    ws = torch.zeros(K.paged_decode_workspace_bytes(d, wl.num_seqs, wl.max_seq_len),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty((wl.num_seqs, d.num_q_heads, d.head_dim), dtype=torch.float32,
                      device="cuda")
    calls = {
        "int8": lambda i: K.paged_decode_int8(d, q8, qs, caches[i % copies], bt, sl,
                                              wl.max_seq_len, w_group=G, workspace=ws, out=out),
        "bf16": lambda i: K.paged_decode_bf16pv(d, q8, qs, caches[i % copies], bt, sl,
                                                wl.max_seq_len, workspace=ws, out=out),
        "uint8w": lambda i: K.paged_decode_uint8w(d, q8, qs, caches[i % copies], bt, sl,
                                                  wl.max_seq_len, w_group=G, workspace=ws,
                                                  out=out),
        "bf16qk": lambda i: K.paged_decode_bf16qk(d, qb, caches[i % copies], bt, sl,
                                                  wl.max_seq_len, w_group=G, workspace=ws,
                                                  out=out),
    }
    res = {}
    for name, fn in calls.items():
        for i in range(3):
            fn(i)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(steps):
                fn(i)
        g.replay()
        runs = []
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            runs.append(1e3 * e0.elapsed_time(e1) / steps)
        key = f"{name}_us" if name in ("uint8w", "bf16qk") else f"{name}_pv_us"
        res[key] = round(float(np.median(runs)), 3)
    res["int8_pv_speedup"] = round(res["bf16_pv_us"] / res["int8_pv_us"], 4)
    res["int8_qk_speedup"] = round(res["bf16qk_us"] / res["int8_pv_us"], 4)
    return res


def time_multi_query(G=32, steps=20, min_rotation_mb=512.0):
    """The MHA configuration's 8 new tokens per sequence (32 heads x 128, 8
    sequences, history ~ U{1024..16384}) decoded as 8 causal queries in one
    paged_decode_ex call (K/V read once), against 8 one-query decode calls
    over the cut sequences; also the bf16-output variant."""
    import numpy as np
    import torch

    import int8_kv_quantized_amd as K
    import workloads as W
    wl = W.cfg5_mha_producer_decode(G)
    nq = 8
    d = K.CacheDesc(wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.num_blocks)
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    base = K.PagedCache.allocate(d)
    K.kv_quantize_write(d, dev(wl.key), dev(wl.value), dev(wl.slot_mapping), base)
    q8, qs = K.kv_quantize_write(d, dev(wl.key[wl.query_token_index]),
                                 dev(wl.value[wl.query_token_index]),
                                 dev(wl.slot_mapping[wl.query_token_index]), base,
                                 query=dev(wl.query))
    copies = max(1, math.ceil(min_rotation_mb * 1e6 / cache_bytes(d)))
    caches = [base] + [K.PagedCache(base.k_cache.clone(), base.v_cache.clone(),
                                    base.k_scale.clone(), base.v_scale.clone())
                       for _ in range(copies - 1)]
    bt, sl = dev(wl.block_tables), dev(wl.seq_lens)
    cut = [dev(wl.seq_lens - (nq - 1 - j)) for j in range(nq)]
    q8j = [q8.view(wl.num_seqs, nq, *q8.shape[1:])[:, j].contiguous() for j in range(nq)]
    qsj = [qs.view(wl.num_seqs, nq, -1)[:, j].contiguous() for j in range(nq)]
    opts = K.DecodeOpts(256, G, 1.0 / math.sqrt(d.head_dim), 0, nq, 0)
    ws = torch.zeros(max(K.paged_decode_ex_workspace_bytes(d, opts, wl.num_seqs, wl.max_seq_len),
                         K.paged_decode_workspace_bytes(d, wl.num_seqs, wl.max_seq_len)),
                     dtype=torch.uint8, device="cuda")
    o32 = torch.empty((wl.num_seqs * nq, d.num_q_heads, d.head_dim), dtype=torch.float32,
                      device="cuda")
    o16 = torch.empty_like(o32, dtype=torch.bfloat16)
    oj = torch.empty((wl.num_seqs, d.num_q_heads, d.head_dim), dtype=torch.float32, device="cuda")

    def multi(i, out):
        K.paged_decode_ex(d, q8, qs, caches[i % copies], bt, sl, wl.max_seq_len,
                          queries_per_seq=nq, w_group=G, out_bf16=out.dtype == torch.bfloat16,
                          workspace=ws, out=out)

    def separate(i):
        for j in range(nq):
            K.paged_decode_int8(d, q8j[j], qsj[j], caches[i % copies], bt, cut[j],
                                wl.max_seq_len, w_group=G, workspace=ws, out=oj)

    res = {}
    for name, fn in (("multi_query_us", lambda i: multi(i, o32)),
                     ("multi_query_bf16_out_us", lambda i: multi(i, o16)),
                     ("separate_calls_us", separate)):
        res[name] = round(_graph_us(fn, steps, reps=5), 3)
    eff = wl.effective_kv_bytes()
    res["multi_query_gbs"] = round(eff / (res["multi_query_us"] * 1e-6) / 1e9, 1)
    res["speedup_vs_separate"] = round(res["separate_calls_us"] / res["multi_query_us"], 3)
    return res


DECODE_SOURCES = ["int8_kv_quantized_amd/csrc/decode.hip", "int8_kv_quantized_amd/csrc/kernels.hpp",
                  "int8_kv_quantized_amd/csrc/device_common.hpp"]
PREFILL_SOURCES = ["int8_kv_quantized_amd/csrc/prefill.hip", "int8_kv_quantized_amd/csrc/kernels.hpp",
                   "int8_kv_quantized_amd/csrc/device_common.hpp"]


def counted_traffic(workload, G, sources=None):
    """HBM bytes per launch of a kernel from the committed FETCH_SIZE /
    WRITE_SIZE counters (profiles/hbm_traffic.json): the decode's partition
    kernel (sources DECODE_SOURCES, the default) or the prefill kernel
    (PREFILL_SOURCES).  None when no record matches the workload, or when the
    kernel's sources changed since the counters were taken."""
    import hashlib
    sources = DECODE_SOURCES if sources is None else sources
    path = ROOT / "profiles" / "hbm_traffic.json"
    if not path.exists():
        return None
    h = hashlib.sha256()
    for s in sources:
        h.update((ROOT / s).read_bytes())
    for rec in json.loads(path.read_text()):
        if (rec.get("workload") == workload and rec.get("w_group") == G
                and rec.get("kernel_sources") == sources
                and rec.get("kernel_sources_sha256") == h.hexdigest()
                and "hbm_bytes_per_launch" in rec):
            return int(rec["hbm_bytes_per_launch"])
    return None


def cpu_baseline(wl, G, seconds):
    """The oracle, single-threaded, on the same decode workload (whole calls)."""
    import numpy as np

    import oracle
    orc = oracle.default()
    cache, q8, qs = orc.fill(wl)
    rows = wl.decode_query_rows()
    q8, qs = q8[rows], qs[rows]
    reps, t0 = 0, time.perf_counter()
    while True:
        orc.paged_decode(q8, qs, cache, wl.block_tables, wl.seq_lens,
                         num_q_heads=wl.num_q_heads, w_group=G)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    gbs = wl.effective_kv_bytes() * reps / el / 1e9
    model = "unknown CPU"
    try:
        with open("/proc/cpuinfo") as f:
            model = next(line.split(":", 1)[1].strip() for line in f
                         if line.startswith("model name"))
    except (OSError, StopIteration):
        pass
    return dict(value=round(gbs, 4), unit="GB/s", cores=1, kind="oracle",
                sample=f"{reps} whole decode calls of {wl.name} ({el:.1f} s, single thread; "
                       f"host has {os.cpu_count()} logical CPUs, {model})")


def host_threads(cap=16):
    """CPUs this process may use, at most ``cap`` (one GPU's share of the host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(cap, n))


def prefill_sample_rows(chunk=2048, n=256, seed=1004):
    """The seeded prefill rows of the CPU leg: the first and last row of every
    32-row tile, plus seeded others up to ``n``."""
    import numpy as np
    starts = np.arange(0, chunk, 32)
    ends = set(starts.tolist()) | set(np.minimum(starts + 31, chunk - 1).tolist())
    rest = np.array(sorted(set(range(chunk)) - ends))
    extra = np.random.default_rng(seed).choice(rest, size=max(0, n - len(ends)), replace=False)
    return np.array(sorted(ends | set(extra.tolist())), np.int32)


def fp64_attention_error(gpu, wl, rows=None):
    """max-abs / mean-abs of GPU outputs against unquantized softmax attention
    over the bf16 inputs, in fp64 (decode: each sequence's newest query over
    its tokens; prefill: the given query rows, causal)."""
    import numpy as np

    import workloads as W
    Hq, Hkv, D = wl.num_q_heads, wl.num_kv_heads, wl.head_dim
    grp = Hq // Hkv
    scale = 1.0 / math.sqrt(D)
    ref = np.zeros(gpu.shape, np.float64)
    qsl = wl.query_start_loc
    for b in range(wl.num_seqs):
        idx = np.nonzero(wl.token_seq == b)[0]
        idx = idx[np.argsort(wl.token_pos[idx], kind="stable")]
        Kf = W.bf16_bits_to_f32(wl.key[idx]).astype(np.float64)
        Vf = W.bf16_bits_to_f32(wl.value[idx]).astype(np.float64)
        if rows is None:   # decode: row b is the sequence's newest query
            qrows, pos, dst = [int(qsl[b + 1]) - 1], [Kf.shape[0] - 1], [b]
        else:
            sel = [i for i, r in enumerate(rows) if qsl[b] <= r < qsl[b + 1]]
            ctx = int(wl.seq_lens[b]) - int(qsl[b + 1] - qsl[b])
            qrows = [int(rows[i]) for i in sel]
            pos = [ctx + r - int(qsl[b]) for r in qrows]
            dst = sel
        if not qrows:
            continue
        Q = W.bf16_bits_to_f32(wl.query[qrows]).astype(np.float64)   # [n, Hq, D]
        pos = np.asarray(pos)
        mask = np.arange(Kf.shape[0])[None, :] > pos[:, None]
        for h in range(Hkv):
            q = Q[:, h * grp:(h + 1) * grp].reshape(-1, D)            # [n*grp, D]
            sc = (q @ Kf[:, h].T) * scale
            sc = sc.reshape(len(qrows), grp, -1)
            sc[np.broadcast_to(mask[:, None, :], sc.shape)] = -np.inf
            sc -= sc.max(axis=-1, keepdims=True)
            pr = np.exp(sc)
            pr /= pr.sum(axis=-1, keepdims=True)
            o = pr.reshape(-1, Kf.shape[0]) @ Vf[:, h]
            ref[dst, h * grp:(h + 1) * grp] = o.reshape(len(qrows), grp, D)
    err = np.abs(gpu.astype(np.float64) - ref)
    return dict(max_abs=float(err.max()), mean_abs=float(err.mean()))


def cpu_leg(args, head, decode_cfgs, prefill_cfg):
    """The CPU-baseline leg: the oracle timed on bounded samples of the
    workloads, and its outputs compared with the GPU outputs taken outside the
    timed regions (max-abs / mean-abs), beside the error of the GPU outputs
    against unquantized fp64 attention."""
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    orc = oracle.default()
    res = {}
    # the headline baseline: whole 16K decode calls, one thread
    res["cpu_baseline"] = cpu_baseline(head["wl"], args.w_group, args.cpu_seconds)
    log(f"cpu baseline: {res['cpu_baseline']}")
    acc = {}

    def decode_acc(wl, outs):
        cache, q8, qs = orc.fill(wl)
        rows = wl.decode_query_rows()
        rec = {}
        for G, gpu in outs.items():
            ref = orc.paged_decode(q8[rows], qs[rows], cache, wl.block_tables, wl.seq_lens,
                                   num_q_heads=wl.num_q_heads, w_group=G)
            e = np.abs(gpu.astype(np.float64) - ref.astype(np.float64))
            rec[f"G{G}"] = dict(vs_oracle_max_abs=float(e.max()),
                                vs_oracle_mean_abs=float(e.mean()),
                                vs_fp64_attention=fp64_attention_error(gpu, wl))
        return rec

    acc[head["wl"].name + "_step"] = decode_acc(head["wl"], {args.w_group: head["out"]})
    for key, (wl, outs) in decode_cfgs.items():
        t0 = time.perf_counter()
        acc[key] = decode_acc(wl, outs)
        log(f"accuracy {key}: {acc[key]} ({time.perf_counter() - t0:.1f} s)")
    if prefill_cfg:
        wl, rows, outs = prefill_cfg["wl"], prefill_cfg["rows"], prefill_cfg["outs"]
        cache, q8, qs = orc.fill(wl)
        threads = host_threads()
        full = np.zeros((wl.query.shape[0], wl.num_q_heads, wl.head_dim), np.float32)
        rec = {}
        for G, gpu in outs.items():
            parts = [rows[i:i + 4] for i in range(0, rows.size, 4)]
            t0 = time.perf_counter()
            with ThreadPoolExecutor(threads) as ex:
                list(ex.map(lambda r: orc.prefix_prefill(q8, qs, wl.query_start_loc, wl.seq_lens,
                                                         cache, wl.block_tables, w_group=G,
                                                         rows=r, out=full), parts))
            el = time.perf_counter() - t0
            e = np.abs(gpu.astype(np.float64) - full[rows].astype(np.float64))
            rec[f"G{G}"] = dict(vs_oracle_max_abs=float(e.max()),
                                vs_oracle_mean_abs=float(e.mean()),
                                vs_fp64_attention=fp64_attention_error(gpu, wl, rows),
                                rows=int(rows.size))
            if G == 32:
                ctx = int(wl.seq_lens[0]) - int(wl.query.shape[0])
                ops = 2 * 2 * wl.head_dim * wl.num_q_heads * int(np.sum(ctx + rows + 1))
                res["cpu_baseline_prefill"] = dict(
                    value=round(ops / el / 1e12, 6), unit="int8 TOPS", cores=threads,
                    kind="oracle",
                    sample=(f"{rows.size} seeded query rows (the first and last row of each "
                            f"32-row tile and seeded others) of {wl.name}, all {wl.num_q_heads} "
                            f"heads, G=32, in {el:.1f} s on {threads} host threads, one row "
                            f"block per thread; whole chunk at this rate: "
                            f"{el * wl.query.shape[0] / rows.size:.0f} s"))
                log(f"cpu baseline prefill: {res['cpu_baseline_prefill']}")
        acc[wl.name.replace("_G32", "")] = rec
        log(f"accuracy prefill: {rec}")
    res["accuracy"] = acc
    return res


def copy_calibration(mb, reps=10):
    """A plain device-to-device copy of known size: its FETCH_SIZE/WRITE_SIZE
    counters give the scale factor for the kernels' byte counters."""
    import torch
    n = int(mb * 1e6) // 16 * 16
    a = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    b = torch.empty(n, dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_per_launch": n, "launches": reps}), flush=True)


def main():
    args = parse_args()
    if args.copy_calibration_mb:
        copy_calibration(args.copy_calibration_mb)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the path has no multi-GPU component).", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    import int8_kv_quantized_amd as K
    import workloads as W
    K.load_library()

    r = time_decode(args)
    wl = r["wl"]
    eff = wl.effective_kv_bytes()
    step_s = r["ms_per_step"] * 1e-3
    value = eff / step_s / 1e9
    achieved = eff / (r["partition_us"] * 1e-6) / 1e9
    call_gbs = eff / (r["decode_us"] * 1e-6) / 1e9
    log(f"decode: call {r['decode_us']:.2f} us ({100 * call_gbs / HBM_PEAK_GBS:.1f}% of peak), "
        f"partition kernel {r['partition_us']:.2f} us ({100 * achieved / HBM_PEAK_GBS:.1f}%), "
        f"producer {r['producer_us']:.2f} us, step {r['ms_per_step'] * 1e3:.2f} us")
    extra = dict(decode_us=round(r["decode_us"], 3),
                 decode_call_frac_hbm=round(call_gbs / HBM_PEAK_GBS, 4),
                 partition_kernel_us=round(r["partition_us"], 3),
                 producer_us=round(r["producer_us"], 3),
                 step_separate_calls_us=round(r["step_separate_us"], 3),
                 effective_kv_bytes=eff, cache_copies_rotated=r["copies"])
    if not args.no_configs:
        # Labelled separately, never the headline: one cache copy re-read by
        # every call, so the K/V largely come from the 256 MB last-level
        # cache instead of HBM.
        warm = time_decode(argparse.Namespace(**{**vars(args), "min_rotation_mb": 0.0,
                                                 "steps": min(args.steps, 100)}),
                           log_prefix="warm: ")
        extra["warm_last_level_cache"] = dict(
            note="one cache copy re-read by every call (K/V resident in the last-level cache)",
            step_us=round(warm["ms_per_step"] * 1e3, 3), decode_us=round(warm["decode_us"], 3),
            partition_kernel_us=round(warm["partition_us"], 3))
    decode_cfgs = {}
    if not args.no_configs:
        configs = {}
        for key, build, step in (
                ("decode_L512", W.cfg1_decode_512, False),
                ("decode_L4096_outlierV", lambda: W.cfg2_decode(4096), False),
                ("decode_L8192_outlierV", lambda: W.cfg2_decode(8192), False),
                ("decode_L16384_outlierV", lambda: W.cfg2_decode(16384), False),
                ("decode_L32768", W.cfg3_decode_32k, False),
                ("decode_batch16_L1K-32K", W.cfg3_decode_batch16, False),
                ("mha_producer_decode_b8", W.cfg5_mha_producer_decode, True)):
            t0 = time.perf_counter()
            cwl = build()
            rec, outs = measure_decode_config(cwl, steps=args.config_steps,
                                              min_rotation_mb=args.min_rotation_mb,
                                              new_tokens_step=step)
            configs[key] = rec
            decode_cfgs[key] = (cwl, outs)
            log(f"config {key}: {rec} ({time.perf_counter() - t0:.1f} s)")
        extra["configs"] = configs
    prefill_cfg = None
    if not args.no_prefill:
        rows = prefill_sample_rows()
        pouts, precs = {}, {}
        for G in (32, 64):
            pf = time_prefill(args.prefill_reps, G, graph=not args.no_graph,
                              min_rotation_mb=args.min_rotation_mb, keep_rows=rows)
            pouts[G] = pf["rows_out"]
            precs[f"G{G}"] = dict(
                us=round(pf["us"], 2), int8_tops=round(pf["tops"], 2),
                frac_int8_peak=round(pf["tops"] / INT8_PEAK_TOPS, 4),
                # the prefill kernel is the call's only launch
                roofline={"bound": "mfma", "achieved": round(pf["tops"], 2),
                          "peak": INT8_PEAK_TOPS, "unit": "int8 TOP/s",
                          "frac": round(pf["tops"] / INT8_PEAK_TOPS, 4),
                          "traffic": counted_traffic(pf["workload"], G, PREFILL_SOURCES),
                          "kernel": f"prefix_prefill_kernel<256,{G}>"})
            log(f"prefill {pf['workload']} G={G}: {pf['us']:.1f} us, {pf['tops']:.1f} int8 TOPS "
                f"({100 * pf['tops'] / INT8_PEAK_TOPS:.1f}% of peak)")
            if G == 32:
                extra.update(prefill_us=round(pf["us"], 2),
                             prefill_int8_tops=round(pf["tops"], 2),
                             prefill_frac_of_int8_peak=round(pf["tops"] / INT8_PEAK_TOPS, 4),
                             prefill_ops=pf["ops"],
                             prefill_cache_copies_rotated=min(pf["cache_copies_rotated"],
                                                              args.prefill_reps))
        extra["prefill"] = precs
        prefill_cfg = dict(wl=W.cfg4_prefill(), rows=rows, outs=pouts)
        if not args.no_pv_ablation:
            pb = time_prefill(args.prefill_reps, graph=not args.no_graph, bf16pv=True,
                              min_rotation_mb=args.min_rotation_mb)
            log(f"prefill BF16-PV ablation: {pb['us']:.1f} us")
            extra["prefill_bf16pv_us"] = round(pb["us"], 2)
            pq = time_prefill(args.prefill_reps, graph=not args.no_graph, bf16qk=True,
                              min_rotation_mb=args.min_rotation_mb)
            log(f"prefill BF16-QK ablation: {pq['us']:.1f} us")
            extra["prefill_bf16qk_us"] = round(pq["us"], 2)
            pu = time_prefill(args.prefill_reps, graph=not args.no_graph, uint8w=True,
                              min_rotation_mb=args.min_rotation_mb)
            log(f"prefill UINT8-W: {pu['us']:.1f} us")
            extra["prefill_uint8w_us"] = round(pu["us"], 2)
    if not args.no_producer_chunks:
        chunks = {}
        for T in (2242, 4096):
            chunks[f"T{T}"] = time_producer_chunk(T)
            log(f"producer chunk T={T}: {chunks[f'T{T}']}")
        extra["producer_chunk"] = chunks
    if not args.no_multi_query:
        mq = time_multi_query(args.w_group)
        log(f"multi-query decode (MHA, 8 seqs x 8 queries): {mq}")
        extra["multi_query_mha_8x8"] = mq
    if not args.no_pv_ablation:
        abl = {}
        for L in (4096, 8192, 16384):
            abl[f"L{L}"] = time_pv_ablation(L)
            log(f"PV ablation L={L}: {abl[f'L{L}']}")
        extra["pv_ablation"] = abl
    cpu = None
    if not args.no_cpu_baseline:
        leg = cpu_leg(args, r, decode_cfgs, prefill_cfg)
        cpu = leg["cpu_baseline"]
        if "cpu_baseline_prefill" in leg:
            extra["cpu_baseline_prefill"] = leg["cpu_baseline_prefill"]
        extra["accuracy"] = leg["accuracy"]
    line = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.num_seqs, "seq_len": wl.max_seq_len,
                   "q_heads": wl.num_q_heads, "kv_heads": wl.num_kv_heads,
                   "head_dim": wl.head_dim, "page_size": 16, "w_group": args.w_group,
                   "partition": 256,
                   "step": ("decode_step_int8 (producer of the new token, with Q, fused "
                            "into paged decode)" if r["fused"] else
                            "kv_quantize_write(new token, with Q) + paged_decode_int8")},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": counted_traffic(wl.name, args.w_group),
                     "kernel": ("paged_decode_partition_kernel<256,32> (the decode's partition "
                                "stage, i8kv_paged_decode_partials), one launch over the whole "
                                "16K history")},
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
