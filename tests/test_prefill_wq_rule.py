"""The prefill kernel's W-code rule against the definition's division (CPU).

The definition ("Implementing INT8 PV MMAC on a gfx936 DCU", section 1):
sW = max W / 127 and Wq = round(W / sW), an IEEE fp32 division with ties
away from zero.  The prefill kernel instead multiplies: inv = 127 * r with r
the hardware reciprocal of max W (within one unit in the last place of
1 / max W), and Wq = the fp32 product W * inv rounded to the nearest integer
by the byte conversion (ties to even).  The two can differ by one code where
W / sW lies next to a half-integer.

On a sample of the 2048-over-16384 chunk (rows at row-tile ends, all 24
heads, the oracle's own W = p~ sV of every visible key, aligned 32-key
groups), this counts the codes the kernel rule changes for each of the three
reciprocals the hardware may return (the correctly rounded one and its two
neighbours) and bounds what the changes do to the output:
|dO[d]| <= sum over changed keys of sW |dWq| |Vq[d]| / l.
Both must stay far below the parity tolerance (max-abs 1e-3).
"""
import numpy as np
import pytest

import workloads as W


def kernel_codes(w, am, r):
    inv = np.float32(np.float32(127.0) * np.float32(r))
    x = (w * inv).astype(np.float32)           # the fp32 product
    return np.rint(x).astype(np.int64)          # nearest, ties to even


def ieee_codes(w, am):
    sw = np.float32(am / np.float32(127.0))
    q = (w / sw).astype(np.float32)   # IEEE fp32 quotient
    return np.where(q >= 0, np.floor(q + np.float32(0.5)), np.ceil(q - np.float32(0.5))).astype(
        np.int64), sw


@pytest.mark.slow
def test_prefill_reciprocal_rule_flips_are_rare_and_bounded(orc):
    wl = W.cfg4_prefill()
    cache, q8, qs = orc.fill(wl)
    qsl, sl, bt = wl.query_start_loc, wl.seq_lens, wl.block_tables
    ctx = int(sl[0]) - int(qsl[1] - qsl[0])
    rows = [0, 31, 1023, 2047]
    total = 0
    flips = {k: 0 for k in ("rn", "up", "down")}
    worst = {k: 0.0 for k in flips}
    for row in rows:
        for head in range(wl.num_q_heads):
            t = orc.prefill_row(q8, qs, qsl, sl, cache, bt, row, head, w_group=32)
            nk = t["nk"]
            keys = np.arange(nk)
            page = bt[0, keys // 16]
            off = keys % 16
            kv = head // (wl.num_q_heads // wl.num_kv_heads)
            sv = cache["v_scale"][page, off, kv]
            vq = cache["v_cache"][page, kv, :, off].astype(np.int64)      # [nk, D]
            w = (t["ptil"] * sv).astype(np.float32)
            # the oracle's own codes are the IEEE rule on these W (sanity)
            dO = {k: np.zeros(wl.head_dim) for k in flips}
            for g0 in range(0, nk, 32):
                gw = w[g0:g0 + 32]
                am = np.float32(gw.max())
                if am == 0:
                    continue
                qi, sw = ieee_codes(gw, am)
                assert np.array_equal(qi, t["Wq"][g0:g0 + 32].astype(np.int64)), (row, head, g0)
                total += gw.size
                r = np.float32(1.0) / am
                for k, rr in (("rn", r), ("up", np.nextafter(r, np.float32(np.inf))),
                              ("down", np.nextafter(r, np.float32(0)))):
                    qk = kernel_codes(gw, am, rr)
                    assert qk.min() >= 0 and qk.max() <= 127
                    d = qk - qi
                    nz = np.nonzero(d)[0]
                    flips[k] += nz.size
                    if nz.size:
                        dO[k] += float(sw) * (d[nz, None] * vq[g0 + nz]).sum(axis=0)
            for k in flips:
                worst[k] = max(worst[k], float(np.abs(dO[k]).max()) / float(t["l"][0]))
    print(f"codes compared: {total}; changed by the reciprocal rule: {flips}; "
          f"largest output change |dO|: {worst}")
    for k in flips:
        assert flips[k] <= 1e-3 * total
        assert worst[k] < 1e-4
