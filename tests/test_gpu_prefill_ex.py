"""The prefill with options (i8kv_prefix_prefill_ex): the PV variant chosen by
an option, and a bf16 output (the attention call of "INT8 KV and INT8 MMAC
attention inference optimisation on a gfx936 DCU", section 3.2, writes bf16).

* pv = int8 / bf16 / uint8 with an fp32 output equals i8kv_prefix_prefill_int8
  / _bf16pv / _uint8w bit for bit (the same kernels);
* the bf16 output equals the call's own fp32 output rounded to bf16 (nearest,
  ties to even; torch's conversion) bit for bit, and the oracle's fp32 output
  rounded to bf16 within one bf16 ulp of |O| plus the fp32 tolerance;
* the fp32 output of every variant agrees with the oracle (max-abs 1e-3,
  mean-abs 1e-4)."""
import numpy as np
import pytest

import workloads as W
from gpu_helpers import assert_bits_equal, assert_close, dev, gpu_fill, oracle_rows, say

pytestmark = pytest.mark.gpu

CASES = [
    dict(name="ex_ragged_d128_g3", seq_lens=(40, 300, 33, 130, 700), new_tokens=(8, 50, 33, 1, 200),
         num_q_heads=6, num_kv_heads=2, head_dim=128),
    dict(name="ex_d256_g6", seq_lens=(600, 300), new_tokens=(100, 37), num_q_heads=24,
         num_kv_heads=4, head_dim=256),
    dict(name="ex_d64_mha", seq_lens=(70, 129), new_tokens=(70, 64), num_q_heads=4,
         num_kv_heads=4, head_dim=64),
]


@pytest.mark.parametrize("G", [32, 64])
@pytest.mark.parametrize("kw", CASES, ids=lambda k: k["name"])
def test_prefill_ex(orc, kw, G):
    import torch

    import int8_kv_quantized_amd as K
    from oracle import ORC_BF16_PV, ORC_UINT8_W
    kw = dict(kw)
    name = kw.pop("name")
    wl = W.make_workload(name, seed=131, kind="prefill", w_group=G, **kw)
    say(f"  prefill_ex case {wl.name} G={G}")
    d, cache, q8, qs = gpu_fill(wl)
    qsl = wl.query_start_loc
    max_q = int((qsl[1:] - qsl[:-1]).max())
    args = (d, q8, qs, dev(qsl), dev(wl.seq_lens), cache, dev(wl.block_tables), max_q)
    plain = {"int8": K.prefix_prefill_int8(*args, w_group=G),
             "bf16": K.prefix_prefill_bf16pv(*args),
             "uint8": K.prefix_prefill_uint8w(*args, w_group=G)}
    ex = {pv: K.prefix_prefill_ex(*args, pv=pv, w_group=G) for pv in plain}
    exb = K.prefix_prefill_ex(*args, pv="int8", w_group=G, out_bf16=True)
    torch.cuda.synchronize()
    for pv in plain:
        assert_bits_equal(ex[pv].cpu().numpy(), plain[pv].cpu().numpy(),
                          f"{wl.name} prefill_ex pv={pv} vs the dedicated call")
    out = plain["int8"].cpu().numpy()
    ob = exb.float().cpu().numpy()
    mine = plain["int8"].to(torch.bfloat16).float().cpu().numpy()
    assert_bits_equal(ob, mine, f"{wl.name} bf16 output vs own fp32 output rounded")
    ocache, oq8, oqs = orc.fill(wl)
    rows = np.arange(out.shape[0], dtype=np.int32)
    for pv, flags in (("int8", 0), ("bf16", ORC_BF16_PV), ("uint8", ORC_UINT8_W)):
        # the BF16-PV ablation rounds W against the running max of each
        # 64-key tile, so its oracle runs 64-key tiles
        g, tile = (64, 64) if pv == "bf16" else (G, 256)
        ref = oracle_rows(lambda **k: orc.prefix_prefill(oq8, oqs, qsl, wl.seq_lens, ocache,
                                                         wl.block_tables, w_group=g, tile=tile,
                                                         flags=flags, **k),
                          rows, np.zeros_like(out))
        assert_close(ex[pv].cpu().numpy(), ref, f"{wl.name} prefill_ex pv={pv} G={g}")
        if pv == "int8":
            refb = orc.round_bf16(ref)
            ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 1e-30))) - 7)
            assert np.all(np.abs(ob - refb) <= ulp + 1e-3), f"{wl.name} bf16 output vs oracle"
