"""The calls captured in HIP graphs (as the benchmark times them) give the
eager result on every replay.

Each call is run eagerly once; the same call on the same buffers is then
captured in a graph and replayed three times, with other eager work and
host synchronizations between the replays, and every replay's output is
compared bit for bit with the eager one (the kernels are deterministic: no
atomics, fixed reduction orders).  The fused step rewrites the newest token's
codes each time, which must also come out unchanged.
"""
import numpy as np
import pytest

import workloads as W
from gpu_helpers import assert_bits_equal, cache_to_np, decode_queries, desc_of, dev, gpu_fill, say

pytestmark = pytest.mark.gpu


def replay_and_check(run, outs, disturb, what):
    import torch
    eager = [o.clone() for o in outs]
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run()                                     # warm the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        run()
    for r in range(3):
        for o in outs:
            o.fill_(float("nan") if o.dtype.is_floating_point else 77)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert_bits_equal(o.cpu().numpy(), e.cpu().numpy(), f"{what} replay {r}")
        disturb()                                 # unrelated eager work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("G", [32, 64])
def test_decode_graph_replay(G):
    import int8_kv_quantized_amd as K
    import torch
    wl = W.make_workload("graph_decode", seq_lens=(700, 300, 1), new_tokens=(1, 1, 1),
                         num_q_heads=24, num_kv_heads=4, head_dim=256, seed=91, w_group=G)
    say(f"  graph replay decode G={G}")
    d, cache, q8, qs = gpu_fill(wl)
    dq8, dqs = decode_queries(q8, qs, wl)
    bt, sl = dev(wl.block_tables), dev(wl.seq_lens)
    S = wl.num_seqs
    ws = torch.zeros(max(K.paged_decode_workspace_bytes(d, S, wl.max_seq_len), 256),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty((S, d.num_q_heads, d.head_dim), dtype=torch.float32, device="cuda")
    other = torch.empty_like(out)
    run = lambda: K.paged_decode_int8(d, dq8, dqs, cache, bt, sl, wl.max_seq_len, w_group=G,
                                      workspace=ws, out=out)
    run()
    torch.cuda.synchronize()
    disturb = lambda: K.paged_decode_int8(d, dq8, dqs * 0.5, cache, bt, sl, wl.max_seq_len,
                                          w_group=G, out=other)
    replay_and_check(run, [out], disturb, f"decode G={G}")


def test_decode_step_graph_replay():
    import int8_kv_quantized_amd as K
    import torch
    wl = W.make_workload("graph_step", seq_lens=(600, 257, 40), new_tokens=(1, 1, 1),
                         num_q_heads=24, num_kv_heads=4, head_dim=256, seed=92)
    say("  graph replay fused decode step")
    d = desc_of(wl)
    is_q = np.zeros(wl.num_tokens, bool)
    is_q[wl.query_token_index] = True
    hist = np.nonzero(~is_q)[0]
    rows = wl.decode_query_rows()
    newest = wl.query_token_index[rows]
    cache = K.PagedCache.allocate(d)
    K.kv_quantize_write(d, dev(wl.key[hist]), dev(wl.value[hist]), dev(wl.slot_mapping[hist]),
                        cache)
    bt, sl = dev(wl.block_tables), dev(wl.seq_lens)
    S = wl.num_seqs
    kn, vn, qn = dev(wl.key[newest]), dev(wl.value[newest]), dev(wl.query[rows])
    ws = torch.zeros(max(K.paged_decode_workspace_bytes(d, S, wl.max_seq_len), 256),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty((S, d.num_q_heads, d.head_dim), dtype=torch.float32, device="cuda")
    q8 = torch.empty((S, d.num_q_heads, d.head_dim), dtype=torch.int8, device="cuda")
    qs = torch.empty((S, d.num_q_heads), dtype=torch.float32, device="cuda")
    run = lambda: K.decode_step_int8(d, kn, vn, qn, cache, bt, sl, wl.max_seq_len, workspace=ws,
                                     out=out, q_int8=q8, q_scale=qs)
    run()
    torch.cuda.synchronize()
    before = cache_to_np(cache)
    other = torch.empty_like(out)
    disturb = lambda: K.paged_decode_int8(d, q8, qs, cache, bt, sl, wl.max_seq_len, out=other)
    replay_and_check(run, [out, q8, qs], disturb, "decode step")
    after = cache_to_np(cache)
    for k in before:
        assert_bits_equal(after[k], before[k], f"decode step {k} after replays")


@pytest.mark.parametrize("G", [32, 64])
def test_prefill_graph_replay(G):
    import int8_kv_quantized_amd as K
    import torch
    wl = W.make_workload("graph_prefill", seq_lens=(600, 130), new_tokens=(100, 130),
                         num_q_heads=24, num_kv_heads=4, head_dim=256, seed=93, kind="prefill",
                         w_group=G)
    say(f"  graph replay prefill G={G}")
    d, cache, q8, qs = gpu_fill(wl)
    qsl = wl.query_start_loc
    max_q = int((qsl[1:] - qsl[:-1]).max())
    loc = (dev(qsl), dev(wl.seq_lens), cache, dev(wl.block_tables), max_q)
    out = torch.empty((q8.shape[0], d.num_q_heads, d.head_dim), dtype=torch.float32,
                      device="cuda")
    other = torch.empty_like(out)
    run = lambda: K.prefix_prefill_int8(d, q8, qs, *loc, w_group=G, out=out)
    run()
    torch.cuda.synchronize()
    disturb = lambda: K.prefix_prefill_int8(d, q8, qs * 2.0, *loc, w_group=G, out=other)
    replay_and_check(run, [out], disturb, f"prefill G={G}")
