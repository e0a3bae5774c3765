"""Pins for the CPU oracle: checks against facts that do not come from the
oracle itself.

Each ``pin_*`` function takes an ``oracle.Oracle`` and raises AssertionError
when the oracle disagrees with what the pages or the mathematics fix:

* worked quantization examples (tests/golden/quantize_ties.txt) and a brute
  force "nearest code, ties away from zero" search over all 255 codes;
* cache layouts re-derived with numpy transposes;
* the integer QK accumulator recomputed with numpy int64 dot products, the
  score chain checked against fp64;
* the softmax probabilities against an fp64 softmax of the same scores;
* W-group quantization against the brute-force nearest code on aligned
  groups; ranges and int32 bounds;
* the output re-assembled from the intermediates (the error decomposition of
  the page "Implementing INT8 PV MMAC on a gfx936 DCU", section 1);
* partition / tile invariance: exact fp64 attention over the dequantized cache
  computed by numpy must equal the oracle's partitioned or tiled result;
* brute force against unquantized fp64 attention within an a-priori bound;
* special cases with closed-form answers (one token, equal scores, one
  dominant score, empty sequence).
* several causal queries per sequence against numpy fp64 causal attention;
* the UINT8-W variant: brute-force nearest codes in [0, 255], group sums
  recomputed with integers, the bound with sW = max / 255;
* the BF16-PV ablation (decode and prefill): W rounded to bf16 exactly as
  torch rounds it, the partition sums / the tile re-assembly recomputed, and
  the bound against unquantized attention;
* the BF16-QK ablation (decode and prefill): bit-identical to the int8 path
  for a bf16 query that is int8 codes times a power of two, exact mode
  against numpy softmax attention of the bf16 query, and the decode bound;
* the rotary embedding against complex multiplication in fp64 (within the
  rounding of two fp32 products and a sum), exact quarter turns and identity
  tables, relative-position invariance of dot products; the producer with
  RoPE against nearest codes of the fp64-rotated vectors.

The mutation tests run the same functions on oracle builds with planted
mistakes and require at least one pin to fail for each.
"""
from __future__ import annotations

from pathlib import Path

import numpy as np

import workloads as W
from oracle import ORC_EXACT, ORC_NO_WQUANT
from refmath import (cache_rows, decode_reference_fp64, prefill_reference_fp64,
                     seq_slots)

GOLDEN = Path(__file__).resolve().parent / "golden"
CODES = np.arange(-127, 128, dtype=np.int64)


# ---------------------------------------------------------------------------
# helpers
# ---------------------------------------------------------------------------
def nearest_code(r: np.ndarray) -> np.ndarray:
    """Brute force: the code in [-127, 127] nearest to each r; ties go to the
    code of larger magnitude (half away from zero)."""
    r = np.asarray(r, np.float64).reshape(-1)
    dist = np.abs(r[:, None] - CODES[None, :].astype(np.float64))
    best = dist.min(axis=1, keepdims=True)
    cand = np.where(dist == best, np.abs(CODES)[None, :], -1)
    pick = cand.argmax(axis=1)
    return CODES[pick]


def check_group_quant(w: np.ndarray, wq: np.ndarray, sw: np.float32, where: str):
    """sW = max W / 127 (fp32) and Wq = nearest code of W / sW (fp32)."""
    w = np.asarray(w, np.float32)
    amax = np.float32(np.abs(w).max()) if w.size else np.float32(0)
    if amax == 0:
        assert sw == 0 and not wq.any(), f"{where}: zero group must give sW=0, Wq=0"
        return
    exp_sw = np.float32(amax) / np.float32(127)
    assert np.float32(sw).view(np.uint32) == exp_sw.view(np.uint32), \
        f"{where}: sW {sw!r} != max/127 {exp_sw!r}"
    r = (w / np.float32(sw)).astype(np.float32)
    exp_q = nearest_code(r)
    assert np.array_equal(wq.astype(np.int64), exp_q), f"{where}: Wq differs from nearest code"
    assert wq.min() >= 0 and wq.max() <= 127, f"{where}: Wq outside [0,127]"
    assert wq.max() == 127, f"{where}: nonzero group without a 127 code"


def tiny_decode(seed=5, seq_lens=(1, 5, 16, 17, 80, 256, 257, 300, 700), Hq=4, Hkv=2,
                D=32, **kw):
    return W.make_workload("tiny_decode", seq_lens=list(seq_lens),
                           new_tokens=[1] * len(seq_lens), num_q_heads=Hq,
                           num_kv_heads=Hkv, head_dim=D, seed=seed, **kw)


def tiny_prefill(seed=9, seq_lens=(40, 300, 33, 130), new=(8, 50, 33, 1), Hq=4, Hkv=2,
                 D=32, **kw):
    return W.make_workload("tiny_prefill", seq_lens=list(seq_lens), new_tokens=list(new),
                           num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, seed=seed,
                           kind="prefill", **kw)


# ---------------------------------------------------------------------------
# quantization
# ---------------------------------------------------------------------------
def pin_quantize_golden(orc):
    n = 0
    for line in (GOLDEN / "quantize_ties.txt").read_text().splitlines():
        if not line.strip() or line.startswith("#"):
            continue
        xs, s, qs = (part.split() for part in line.split("|"))
        x = np.array([float(v) for v in xs], np.float32)
        assert np.array_equal(W.bf16_bits_to_f32(W.f32_to_bf16_bits(x)), x)
        q, sc = orc.quantize(x)
        assert sc == np.float32(float(s[0])), f"golden scale {sc} != {s[0]}"
        assert np.array_equal(q.astype(int), np.array([int(v) for v in qs])), \
            f"golden codes {q.tolist()} != {qs}"
        n += 1
    assert n >= 5


def pin_quantize_bruteforce(orc, n_vec=240, seed=11):
    rng = np.random.default_rng(seed)
    for t in range(n_vec):
        D = int(rng.choice([16, 128, 256]))
        kind = t % 4
        if kind == 0:
            x = rng.standard_normal(D).astype(np.float32)
        elif kind == 1:     # exact ties: (k + 1/2) * 2^e with one element at 127 * 2^e
            e = float(2.0 ** rng.integers(-20, 20))
            k = rng.integers(-126, 127, D).astype(np.float64) + 0.5 * rng.integers(0, 2, D)
            k[rng.integers(D)] = 127.0 * (1 if rng.random() < 0.5 else -1)
            x = (k * e).astype(np.float32)
        elif kind == 2:     # tiny magnitudes: scales fall into the subnormal range
            x = (rng.standard_normal(D) * 1e-38).astype(np.float32)
        else:               # wide dynamic range
            x = (rng.standard_normal(D) * 10.0 ** rng.uniform(-30, 30, D)).astype(np.float32)
        x = W.bf16_bits_to_f32(W.f32_to_bf16_bits(x))
        q, s = orc.quantize(x)
        amax = np.float32(np.abs(x).max())
        if amax == 0:
            assert s == 0 and not q.any()
            continue
        exp_s = amax / np.float32(127)
        assert s.view(np.uint32) == exp_s.view(np.uint32), "scale must be amax/127 in fp32"
        r = (x / s).astype(np.float32)
        assert np.array_equal(q.astype(np.int64), nearest_code(r)), "codes not nearest/ties-away"
        assert abs(int(q[np.argmax(np.abs(x))])) == 127
        assert q.min() >= -127
        err = np.abs(q.astype(np.float64) * s - x.astype(np.float64))
        assert np.all(err <= s * (0.5 + 1e-5)), "dequantization error above half a step"


# ---------------------------------------------------------------------------
# producer / layout
# ---------------------------------------------------------------------------
def pin_cache_layout(orc):
    wl = W.make_workload("layout", seq_lens=[37, 16, 1, 70], new_tokens=[1] * 4,
                         num_q_heads=4, num_kv_heads=2, head_dim=64, seed=21)
    rng = np.random.default_rng(3)
    T = wl.num_tokens
    slots = wl.slot_mapping.copy()
    skip = rng.choice(T, 6, replace=False)
    slots[skip] = -1
    qry = W.f32_to_bf16_bits(rng.standard_normal((T, 4, 64), dtype=np.float32))
    cache = orc.empty_cache(wl.num_blocks, 2, 64)
    q8, qs = orc.kv_quantize_write(wl.key, wl.value, slots, cache, num_q_heads=4, query=qry)
    K, V, sK, sV = cache_rows(cache)
    written = np.zeros(K.shape[0], bool)
    for t in range(T):
        for h in range(4):
            qq, ss = orc.quantize(W.bf16_bits_to_f32(qry[t, h]))
            assert np.array_equal(q8[t, h], qq) and qs[t, h] == ss, "query codes/scale"
        if slots[t] < 0:
            continue
        written[slots[t]] = True
        for h in range(2):
            kq, ks = orc.quantize(W.bf16_bits_to_f32(wl.key[t, h]))
            vq, vs = orc.quantize(W.bf16_bits_to_f32(wl.value[t, h]))
            assert np.array_equal(K[slots[t], h], kq), f"K layout, token {t} head {h}"
            assert np.array_equal(V[slots[t], h], vq), f"V layout, token {t} head {h}"
            assert sK[slots[t], h] == ks and sV[slots[t], h] == vs, "scale layout"
    assert not K[~written].any() and not V[~written].any(), "write outside its slot"
    assert not sK[~written].any() and not sV[~written].any(), "scale write outside its slot"


# ---------------------------------------------------------------------------
# rotary position embedding in the producer
# ---------------------------------------------------------------------------
U32 = 2.0 ** -24     # unit roundoff of fp32


def _rotate_complex(x, pos, cs):
    """fp64 reference: the first R dims as R/2 complex numbers
    z_j = x[j] + i x[j + R/2], each multiplied by c + i s from the table
    (the rotate-half pairing); returns (rotated, per-element error bound of a
    product/product/difference evaluation in fp32)."""
    x = np.asarray(x, np.float64)
    R = cs.shape[1]
    h = R // 2
    c = cs[pos, :h].astype(np.float64)
    s = cs[pos, h:].astype(np.float64)
    z = (x[:, :h] + 1j * x[:, h:R]) * (c + 1j * s)
    out = x.copy()
    out[:, :h], out[:, h:R] = z.real, z.imag
    mag = np.abs(x[:, :h] * c) + np.abs(x[:, h:R] * s)
    mag2 = np.abs(x[:, h:R] * c) + np.abs(x[:, :h] * s)
    bound = np.zeros_like(x)
    bound[:, :h], bound[:, h:R] = 2.001 * U32 * mag, 2.001 * U32 * mag2
    return out, bound


def pin_rope_rotation(orc, seed=41):
    """The rotation against complex multiplication in fp64 (within the fp32
    rounding of two products and one sum), on random-angle and standard
    tables, full and partial rotary dims; dims past R unchanged; the identity
    table leaves every bit; relative-position invariance of dot products."""
    rng = np.random.default_rng(seed)
    for D, R in ((64, 64), (128, 64), (256, 256), (32, 8)):
        for table in ("random", "standard"):
            P = 300
            cs = (W.random_cos_sin(rng, P, R) if table == "random"
                  else W.rope_cos_sin(P, R))
            x = W.bf16_bits_to_f32(W.f32_to_bf16_bits(
                rng.standard_normal((40, D), dtype=np.float32)))
            pos = rng.integers(0, P, 40).astype(np.int32)
            got = orc.rope_rotate(x, pos, cs)
            ref, bound = _rotate_complex(x, pos, cs)
            err = np.abs(got.astype(np.float64) - ref)
            assert np.all(err <= bound), \
                f"rotation (D={D}, R={R}, {table}) off by {float((err - bound).max())}"
            assert np.array_equal(got[:, R:], x[:, R:]), "dims past the rotary part changed"
    # identity table: cos 1, sin 0
    x = rng.standard_normal((8, 128), dtype=np.float32)
    cs = np.concatenate([np.ones((5, 32), np.float32), np.zeros((5, 32), np.float32)], 1)
    assert np.array_equal(orc.rope_rotate(x, np.arange(8, dtype=np.int32) % 5, cs), x)
    # a quarter turn: cos 0, sin 1 maps (a, b) -> (-b, a) exactly
    cs = np.concatenate([np.zeros((1, 32), np.float32), np.ones((1, 32), np.float32)], 1)
    got = orc.rope_rotate(x, np.zeros(8, np.int32), cs)
    assert np.array_equal(got[:, :32], -x[:, 32:64]) and np.array_equal(got[:, 32:64], x[:, :32])
    # relative positions: <R_p q, R_n k> depends on p - n only
    R, P = 128, 4096
    cs = W.rope_cos_sin(P, R)
    q = rng.standard_normal((1, R)).astype(np.float32)
    k = rng.standard_normal((1, R)).astype(np.float32)
    for p, n, shift in ((7, 3, 1000), (2000, 1, 2095), (50, 50, 9)):
        d0 = float(orc.rope_rotate(q, np.array([p], np.int32), cs)[0].astype(np.float64)
                   @ orc.rope_rotate(k, np.array([n], np.int32), cs)[0])
        d1 = float(orc.rope_rotate(q, np.array([p + shift], np.int32), cs)[0].astype(np.float64)
                   @ orc.rope_rotate(k, np.array([n + shift], np.int32), cs)[0])
        assert abs(d0 - d1) <= 2e-3 * (1 + abs(d0)), f"relative position ({p},{n}) {d0} vs {d1}"
    # out-of-range positions are rejected
    try:
        orc.rope_rotate(x, np.full(8, 5, np.int32), cs[:5])
    except ValueError:
        pass
    else:
        raise AssertionError("position past the table accepted")


def pin_rope_producer(orc, seed=43):
    """The producer with RoPE: Q and K codes are the nearest codes of the
    rotated (fp64 complex reference) vectors within the fp32 rounding of the
    rotation; V and the slots are those of the plain producer; an identity
    table reproduces the plain producer bit for bit."""
    rng = np.random.default_rng(seed)
    for D, R in ((64, 64), (128, 32)):
        wl = W.make_workload("rope", seq_lens=[37, 16, 1, 70], new_tokens=[1] * 4,
                             num_q_heads=4, num_kv_heads=2, head_dim=D, seed=seed + D)
        T = wl.num_tokens
        qry = W.f32_to_bf16_bits(rng.standard_normal((T, 4, D), dtype=np.float32))
        P = 128
        cs = W.random_cos_sin(rng, P, R)
        pos = rng.integers(0, P, T).astype(np.int32)
        plain = orc.empty_cache(wl.num_blocks, 2, D)
        q8p, qsp = orc.kv_quantize_write(wl.key, wl.value, wl.slot_mapping, plain,
                                         num_q_heads=4, query=qry)
        cache = orc.empty_cache(wl.num_blocks, 2, D)
        q8, qs = orc.kv_quantize_write_rope(wl.key, wl.value, wl.slot_mapping, pos, cs, cache,
                                            num_q_heads=4, query=qry)
        for name in ("v_cache", "v_scale"):
            assert np.array_equal(cache[name], plain[name]), f"{name} must not be rotated"
        K, _, sK, _ = cache_rows(cache)
        for t in range(T):
            for h, (codes, sc, src) in enumerate(
                    [(q8[t, j], qs[t, j], qry[t, j]) for j in range(4)]
                    + [(K[wl.slot_mapping[t], j], sK[wl.slot_mapping[t], j], wl.key[t, j])
                       for j in range(2)]):
                x = W.bf16_bits_to_f32(src)[None]
                ref, bound = _rotate_complex(x, pos[t:t + 1], cs)
                ref, bound = ref[0], bound[0]
                amax = np.abs(ref).max()
                exp_s = amax / 127
                assert abs(float(sc) - exp_s) <= 1e-6 * exp_s + bound.max() / 127, \
                    f"scale of token {t} vector {h}"
                # the code is the nearest one, up to a tie the rotation's rounding may decide
                r = ref / np.float64(sc)
                slack = bound / np.float64(sc) + 2e-6 * np.abs(r) + 1e-9
                assert np.all(np.abs(codes.astype(np.float64) - r) <= 0.5 + slack), \
                    f"code of token {t} vector {h} not nearest to the rotated value"
        # identity table == plain producer
        ident = np.concatenate([np.ones((P, R // 2), np.float32),
                                np.zeros((P, R // 2), np.float32)], 1)
        cache_i = orc.empty_cache(wl.num_blocks, 2, D)
        q8i, qsi = orc.kv_quantize_write_rope(wl.key, wl.value, wl.slot_mapping, pos, ident,
                                              cache_i, num_q_heads=4, query=qry)
        assert np.array_equal(q8i, q8p) and np.array_equal(qsi, qsp), "identity table, Q"
        for name in plain:
            assert np.array_equal(cache_i[name], plain[name]), f"identity table, {name}"


# ---------------------------------------------------------------------------
# decode
# ---------------------------------------------------------------------------
def _softmax64(s):
    s = np.asarray(s, np.float64)
    e = np.exp(s - s.max())
    return e / e.sum()


def pin_decode_trace(orc, G=32, seed=5):
    wl = tiny_decode(seed=seed)
    cache, q8, qs = orc.fill(wl)
    K, V, sK, sV = cache_rows(cache)
    D, grp = wl.head_dim, wl.num_q_heads // wl.num_kv_heads
    scale = wl.softmax_scale
    for b in range(wl.num_seqs):
        for h in range(wl.num_q_heads):
            tr = orc.decode_head(q8, qs, cache, wl.block_tables, wl.seq_lens, b, h, w_group=G)
            L = int(wl.seq_lens[b])
            sl = seq_slots(wl, b)
            kv = h // grp
            acc = K[sl, kv].astype(np.int64) @ q8[b, h].astype(np.int64)
            assert np.array_equal(tr["acc"].astype(np.int64), acc), f"QK acc (seq {b}, head {h})"
            assert np.abs(acc).max() <= D * 127 * 127
            s64 = acc * np.float64(qs[b, h]) * sK[sl, kv].astype(np.float64) * np.float64(scale)
            assert np.all(np.abs(tr["s"] - s64) <= 2e-7 * np.abs(s64) + 1e-30), "score chain"
            o_rec = np.zeros_like(tr["o"])
            for p in range(-(-L // 256)):
                i0, i1 = 256 * p, min(L, 256 * p + 256)
                sp = tr["s"][i0:i1].astype(np.float64)
                assert tr["m"][p] == tr["s"][i0:i1].max(), "partition max"
                P64 = _softmax64(sp)
                tol = 1e-6 * (1 + np.abs(sp - sp.max())) * P64 + 1e-45
                assert np.all(np.abs(tr["P"][i0:i1] - P64) <= tol), "partition softmax"
                lsum = np.exp(sp - sp.max()).sum()
                assert abs(tr["l"][p] - lsum) <= 1e-6 * lsum, "partition exp-sum"
                Wexp = (tr["P"][i0:i1] * sV[sl[i0:i1], kv]).astype(np.float32)
                assert np.array_equal(tr["W"][i0:i1], Wexp), "W = P * sV"
                for g0 in range(i0, i1, G):
                    g1 = min(i1, g0 + G)
                    check_group_quant(tr["W"][g0:g1], tr["Wq"][g0:g1], tr["sW"][g0 // G],
                                      f"decode seq {b} head {h} group {g0 // G}")
                    part = tr["Wq"][g0:g1].astype(np.int64) @ V[sl[g0:g1], kv].astype(np.int64)
                    assert np.abs(part).max(initial=0) <= G * 127 * 127
                    o_rec[p] += np.float64(tr["sW"][g0 // G]) * part
                # error decomposition within the partition (PV article, section 1)
                Porig = tr["P"][i0:i1].astype(np.float64)
                tok = np.nonzero(wl.token_seq == b)[0]
                tok = tok[np.argsort(wl.token_pos[tok])][i0:i1]
                Vorig = W.bf16_bits_to_f32(wl.value[tok, kv]).astype(np.float64)
                sVp = sV[sl[i0:i1], kv].astype(np.float64)
                Vq = V[sl[i0:i1], kv].astype(np.float64)
                eV = Vorig - sVp[:, None] * Vq
                sW_tok = np.repeat(tr["sW"][i0 // G:-(-i1 // G)].astype(np.float64), G)
                sW_tok = sW_tok[:i1 - i0]
                eW = Porig * sVp - sW_tok * tr["Wq"][i0:i1]
                lhs = Porig @ Vorig - o_rec[p]
                rhs = Porig @ eV + eW @ Vq
                assert np.allclose(lhs, rhs, rtol=0, atol=1e-12 * (1 + np.abs(lhs).max()))
            assert np.allclose(tr["o"], o_rec, rtol=1e-12, atol=1e-15), "partition output"
            m = tr["m"].astype(np.float64)
            w = tr["l"].astype(np.float64) * np.exp(m - m.max())
            O = (w[:, None] * o_rec).sum(0) / w.sum()
            assert np.all(np.abs(tr["out"] - O) <= 1e-6 * (np.abs(O) + 1e-3)), "LSE merge"


def pin_decode_bruteforce(orc, G=32, seed=6):
    """Against unquantized fp64 attention, within the bound built from the
    rounding bounds |eV| <= sV/2 and |eW| <= sW/2 plus the QK term."""
    wl = tiny_decode(seed=seed, seq_lens=(1, 7, 16, 33, 100, 256, 300, 520))
    cache, q8, qs = orc.fill(wl)
    K, V, sK, sV = cache_rows(cache)
    ref = decode_reference_fp64(wl)
    grp = wl.num_q_heads // wl.num_kv_heads
    worst = 0.0
    for b in range(wl.num_seqs):
        L = int(wl.seq_lens[b])
        big = 256 * -(-L // 256)   # one partition covering everything
        for h in range(wl.num_q_heads):
            kv = h // grp
            tr = orc.decode_head(q8, qs, cache, wl.block_tables, wl.seq_lens, b, h,
                                 w_group=G, partition=big)
            sl = seq_slots(wl, b)
            tok = np.nonzero(wl.token_seq == b)[0]
            tok = tok[np.argsort(wl.token_pos[tok])]
            Vorig = W.bf16_bits_to_f32(wl.value[tok, kv]).astype(np.float64)
            Korig = W.bf16_bits_to_f32(wl.key[tok, kv]).astype(np.float64)
            qorig = W.bf16_bits_to_f32(wl.query[wl.decode_query_rows()[b], h]).astype(np.float64)
            Pe = _softmax64(Korig @ qorig / np.sqrt(wl.head_dim))
            P = tr["P"].astype(np.float64)
            sVt = sV[sl, kv].astype(np.float64)
            sWt = np.repeat(tr["sW"].astype(np.float64), G)[:L]
            Vq = np.abs(V[sl, kv].astype(np.float64))
            bound = (np.abs(Pe - P) @ np.abs(Vorig) + (P * sVt / 2).sum()
                     + (sWt / 2 * (1 + 1e-6)) @ Vq + 1e-6)
            err = np.abs(tr["out"] - ref[b, h])
            assert np.all(err <= bound), f"decode seq {b} head {h}: error above bound"
            worst = max(worst, float((err / bound).max()))
            out_part = orc.decode_head(q8, qs, cache, wl.block_tables, wl.seq_lens, b, h,
                                       w_group=G)["out"]
            assert np.abs(out_part - ref[b, h]).max() < 0.05, "gross error vs fp64 attention"
    return worst


def nearest_code_u8(r: np.ndarray) -> np.ndarray:
    """Brute force: the code in [0, 255] nearest to each r >= 0, ties up."""
    r = np.asarray(r, np.float64).reshape(-1)
    codes = np.arange(256, dtype=np.int64)
    dist = np.abs(r[:, None] - codes[None, :].astype(np.float64))
    best = dist.min(axis=1, keepdims=True)
    return np.where(dist == best, codes[None, :], -1).max(axis=1)


def pin_quantize_w_u8(orc, seed=14):
    """UINT8 W groups: sW = max W / 255 in fp32, codes the brute-force nearest
    of W / sW (fp32) in [0, 255] with ties up, 255 present, zero group -> 0."""
    rng = np.random.default_rng(seed)
    for t in range(300):
        n = int(rng.choice([1, 7, 32, 64]))
        kind = t % 3
        if kind == 0:
            w = rng.random(n).astype(np.float32) * np.float32(10.0 ** rng.uniform(-8, 0))
        elif kind == 1:  # exact ties: (k + 1/2) * 2^e with a 255 * 2^e maximum
            e = float(2.0 ** rng.integers(-20, 0))
            k = rng.integers(0, 255, n).astype(np.float64) + 0.5 * rng.integers(0, 2, n)
            k[rng.integers(n)] = 255.0
            w = (k * e).astype(np.float32)
        else:
            w = np.zeros(n, np.float32)
            if n > 1:
                w[rng.integers(n)] = np.float32(rng.random())
        q, sw = orc.quantize_w_u8(w)
        amax = np.float32(w.max())
        if amax == 0:
            assert sw == 0 and not q.any(), "zero group must give sW = 0, Wq = 0"
            continue
        assert sw.view(np.uint32) == (amax / np.float32(255)).view(np.uint32), "sW != max/255"
        r = (w / sw).astype(np.float32)
        assert np.array_equal(q.astype(np.int64), nearest_code_u8(r)), "u8 codes not nearest/ties up"
        assert q.max() == 255, "non-zero group without a 255 code"


def pin_decode_uint8_w(orc, G=32, seed=15):
    """The UINT8-W decode: everything before W equals the int8 path; Wq are
    the brute-force nearest codes of W / sW on aligned groups; o is
    sum_g sW * (Wq . Vq) recomputed with numpy int64; the output stays within
    the unquantized-attention bound with the sW / 2 term (sW = max / 255),
    and its error is smaller than the int8 path's on average."""
    from oracle import ORC_UINT8_W
    wl = tiny_decode(seed=seed, seq_lens=(1, 17, 64, 256, 300, 700))
    cache, q8, qs = orc.fill(wl)
    K, V, sK, sV = cache_rows(cache)
    ref = decode_reference_fp64(wl)
    grp = wl.num_q_heads // wl.num_kv_heads
    err8 = err_u = 0.0
    for b in range(wl.num_seqs):
        L = int(wl.seq_lens[b])
        sl = seq_slots(wl, b)
        for h in range(wl.num_q_heads):
            kv = h // grp
            tu = orc.decode_head(q8, qs, cache, wl.block_tables, wl.seq_lens, b, h, w_group=G,
                                 flags=ORC_UINT8_W)
            t8 = orc.decode_head(q8, qs, cache, wl.block_tables, wl.seq_lens, b, h, w_group=G)
            for k in ("s", "P", "W", "m", "l"):
                assert np.array_equal(tu[k], t8[k]), f"uint8-W changed {k}"
            wq = tu["Wq"].view(np.uint8).astype(np.int64)
            vq = V[sl, kv].astype(np.int64)
            for pp in range(-(-L // 256)):
                i0, i1 = 256 * pp, min(L, 256 * pp + 256)
                o = np.zeros(wl.head_dim)
                for g0 in range(i0, i1, G):
                    g1 = min(i1, g0 + G)
                    w = tu["W"][g0:g1]
                    sw = tu["sW"][g0 // G]
                    exp_sw = np.float32(w.max()) / np.float32(255) if w.max() > 0 else np.float32(0)
                    assert sw.view(np.uint32) == np.float32(exp_sw).view(np.uint32), "group sW"
                    if sw > 0:
                        r = (w / sw).astype(np.float32)
                        assert np.array_equal(wq[g0:g1], nearest_code_u8(r)), "group codes"
                    o += np.float64(sw) * (wq[g0:g1] @ vq[g0:g1]).astype(np.float64)
                assert np.allclose(tu["o"][pp], o, rtol=1e-12, atol=1e-12), "o != sum sW Wq.Vq"
            big = 256 * -(-L // 256)
            t1 = orc.decode_head(q8, qs, cache, wl.block_tables, wl.seq_lens, b, h, w_group=G,
                                 partition=big, flags=ORC_UINT8_W)
            tok = np.nonzero(wl.token_seq == b)[0]
            tok = tok[np.argsort(wl.token_pos[tok])]
            Vorig = W.bf16_bits_to_f32(wl.value[tok, kv]).astype(np.float64)
            Korig = W.bf16_bits_to_f32(wl.key[tok, kv]).astype(np.float64)
            qorig = W.bf16_bits_to_f32(wl.query[wl.decode_query_rows()[b], h]).astype(np.float64)
            Pe = _softmax64(Korig @ qorig / np.sqrt(wl.head_dim))
            P = t1["P"].astype(np.float64)
            sVt = sV[sl, kv].astype(np.float64)
            sWt = np.repeat(t1["sW"].astype(np.float64), G)[:L]
            bound = (np.abs(Pe - P) @ np.abs(Vorig) + (P * sVt / 2).sum()
                     + (sWt / 2 * (1 + 1e-6)) @ np.abs(vq) + 1e-6)
            err = np.abs(t1["out"] - ref[b, h])
            assert np.all(err <= bound), f"uint8-W decode seq {b} head {h}: error above bound"
            err_u += np.abs(tu["out"] - ref[b, h]).mean()
            err8 += np.abs(t8["out"] - ref[b, h]).mean()
    assert err_u < err8, f"uint8 W not more accurate on average ({err_u} vs {err8})"


def pin_decode_multi_query(orc, seed=16):
    """Several causal queries per sequence: with ORC_EXACT each query row must
    equal exact fp64 softmax attention, computed here with numpy, over the
    dequantized keys 0 .. its position (L - nq + j); a query past the
    sequence start (L < nq) gives zeros; nq = 1 is the plain decode."""
    wl = W.make_workload("multi", seq_lens=[5, 257, 300, 520], new_tokens=[5, 8, 8, 8],
                         num_q_heads=4, num_kv_heads=2, head_dim=32, seed=seed)
    cache, q8, qs = orc.fill(wl)
    K, V, sK, sV = cache_rows(cache)
    nq = 8
    S = wl.num_seqs
    # rows s*nq + j: the newest 8 query rows of each sequence (sequence 0 has 5)
    q8m = np.zeros((S * nq, 4, 32), np.int8)
    qsm = np.zeros((S * nq, 4), np.float32)
    for b in range(S):
        rows = np.arange(wl.query_start_loc[b], wl.query_start_loc[b + 1])
        q8m[b * nq + nq - len(rows): (b + 1) * nq] = q8[rows]
        qsm[b * nq + nq - len(rows): (b + 1) * nq] = qs[rows]
    out = orc.paged_decode_multi(q8m, qsm, cache, wl.block_tables, wl.seq_lens, num_q_heads=4,
                                 queries_per_seq=nq, flags=ORC_EXACT)
    scale = wl.softmax_scale
    for b in range(S):
        L = int(wl.seq_lens[b])
        sl = seq_slots(wl, b)
        for j in range(nq):
            pos = L - nq + j
            for h in range(4):
                kv = h // 2
                o = out[b * nq + j, h]
                if pos < 0:
                    assert not o.any(), "a query before the sequence start must give zeros"
                    continue
                k = K[sl[:pos + 1], kv].astype(np.float64) * sK[sl[:pos + 1], kv, None]
                v = V[sl[:pos + 1], kv].astype(np.float64) * sV[sl[:pos + 1], kv, None]
                qv = q8m[b * nq + j, h].astype(np.float64) * np.float64(qsm[b * nq + j, h])
                ref = _softmax64(k @ qv * np.float64(scale)) @ v
                assert np.abs(o - ref).max() <= 1e-5 * (1 + np.abs(ref).max()), \
                    f"multi-query row (seq {b}, query {j}, head {h})"
    one = orc.paged_decode_multi(q8m[nq - 1::nq], qsm[nq - 1::nq], cache, wl.block_tables,
                                 wl.seq_lens, num_q_heads=4, queries_per_seq=1)
    ref1 = orc.paged_decode(q8m[nq - 1::nq], qsm[nq - 1::nq], cache, wl.block_tables,
                            wl.seq_lens, num_q_heads=4)
    assert np.array_equal(one, ref1), "nq = 1 must be the plain decode"


def pin_bf16_rounding(orc, seed=13):
    """The oracle's bf16 rounding equals torch's float -> bfloat16 conversion
    (nearest, ties to even) on random values, exact ties with even and odd
    kept bits, neighbours of ties, subnormals and large values."""
    import torch
    rng = np.random.default_rng(seed)
    hi = rng.integers(0, 0x7f7f, 4000, dtype=np.uint32) << 16
    bits = np.concatenate([
        rng.integers(0, 0x7f7fffff, 4000, dtype=np.uint32),
        hi | 0x8000, hi | 0x7fff, hi | 0x8001, (hi & 0x00ff0000) | rng.integers(0, 1 << 16, 4000, dtype=np.uint32)])
    x = bits.view(np.float32)
    x = np.concatenate([x, -x])
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).to(torch.float32).numpy()
    got = orc.round_bf16(x)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), \
        f"bf16 rounding differs on {int((got != ref).sum())} values"


def pin_decode_bf16_pv(orc, seed=12):
    """The BF16-PV ablation (decode): W = P * sV rounded to bf16 by torch's
    own conversion (nearest, ties to even) must equal the oracle's W; each
    partition's o must be sum W * Vq (numpy, fp64); the output stays within
    the unquantized-fp64 bound with the bf16 rounding term 2^-9 W |Vq| in
    place of the W-group term; everything before W equals the int8 path."""
    import torch
    from oracle import ORC_BF16_PV
    wl = tiny_decode(seed=seed, seq_lens=(1, 9, 40, 256, 300, 600))
    cache, q8, qs = orc.fill(wl)
    K, V, sK, sV = cache_rows(cache)
    ref = decode_reference_fp64(wl)
    grp = wl.num_q_heads // wl.num_kv_heads
    for b in range(wl.num_seqs):
        L = int(wl.seq_lens[b])
        sl = seq_slots(wl, b)
        for h in range(wl.num_q_heads):
            kv = h // grp
            tr = orc.decode_head(q8, qs, cache, wl.block_tables, wl.seq_lens, b, h,
                                 flags=ORC_BF16_PV)
            t8 = orc.decode_head(q8, qs, cache, wl.block_tables, wl.seq_lens, b, h)
            for k in ("s", "P", "m", "l"):
                assert np.array_equal(tr[k], t8[k]), f"bf16-PV changed {k} (seq {b} head {h})"
            w32 = (t8["P"] * sV[sl, kv]).astype(np.float32)
            wb = torch.from_numpy(w32).to(torch.bfloat16).to(torch.float32).numpy()
            assert np.array_equal(tr["W"], wb), f"W not bf16-rounded (seq {b} head {h})"
            vq = V[sl, kv].astype(np.float64)
            for pp in range(-(-L // 256)):
                i0, i1 = 256 * pp, min(L, 256 * pp + 256)
                o = wb[i0:i1].astype(np.float64) @ vq[i0:i1]
                assert np.allclose(tr["o"][pp], o, rtol=1e-12, atol=1e-12), "o != sum W Vq"
            # one partition: bound against unquantized fp64 attention
            big = 256 * -(-L // 256)
            t1 = orc.decode_head(q8, qs, cache, wl.block_tables, wl.seq_lens, b, h,
                                 partition=big, flags=ORC_BF16_PV)
            tok = np.nonzero(wl.token_seq == b)[0]
            tok = tok[np.argsort(wl.token_pos[tok])]
            Vorig = W.bf16_bits_to_f32(wl.value[tok, kv]).astype(np.float64)
            Korig = W.bf16_bits_to_f32(wl.key[tok, kv]).astype(np.float64)
            qorig = W.bf16_bits_to_f32(wl.query[wl.decode_query_rows()[b], h]).astype(np.float64)
            Pe = _softmax64(Korig @ qorig / np.sqrt(wl.head_dim))
            P = t1["P"].astype(np.float64)
            sVt = sV[sl, kv].astype(np.float64)
            bound = (np.abs(Pe - P) @ np.abs(Vorig) + (P * sVt / 2).sum()
                     + (2.0 ** -9 * P * sVt * (1 + 1e-6)) @ np.abs(vq) + 1e-6)
            err = np.abs(t1["out"] - ref[b, h])
            assert np.all(err <= bound), f"bf16-PV decode seq {b} head {h}: error above bound"


def pin_decode_partition_invariance(orc, G=32, seed=8):
    wl = tiny_decode(seed=seed, seq_lens=(300, 700, 1000, 257, 513))
    cache, q8, qs = orc.fill(wl)
    K, V, sK, sV = cache_rows(cache)
    ex = ORC_EXACT | ORC_NO_WQUANT
    o256 = orc.paged_decode(q8, qs, cache, wl.block_tables, wl.seq_lens,
                            num_q_heads=wl.num_q_heads, w_group=G, flags=ex)
    obig = orc.paged_decode(q8, qs, cache, wl.block_tables, wl.seq_lens,
                            num_q_heads=wl.num_q_heads, w_group=G, partition=1024, flags=ex)
    # exact softmax attention over the dequantized cache, written directly
    grp = wl.num_q_heads // wl.num_kv_heads
    ref = np.zeros_like(o256, dtype=np.float64)
    for b in range(wl.num_seqs):
        sl = seq_slots(wl, b)
        for h in range(wl.num_q_heads):
            kv = h // grp
            acc = K[sl, kv].astype(np.int64) @ q8[b, h].astype(np.int64)
            s = acc * np.float64(qs[b, h]) * sK[sl, kv].astype(np.float64) * wl.softmax_scale
            p = _softmax64(s)
            ref[b, h] = (p * sV[sl, kv].astype(np.float64)) @ V[sl, kv].astype(np.float64)
    tol = 1e-6 * (np.abs(ref) + 1e-3)
    assert np.all(np.abs(o256 - ref) <= tol), "partitioned exact decode != single softmax"
    assert np.all(np.abs(obig - ref) <= tol), "single-partition exact decode != softmax"
    # quantized: partition size changes only fp32 rounding (Wq tie flips)
    q256 = orc.paged_decode(q8, qs, cache, wl.block_tables, wl.seq_lens,
                            num_q_heads=wl.num_q_heads, w_group=G)
    qbig = orc.paged_decode(q8, qs, cache, wl.block_tables, wl.seq_lens,
                            num_q_heads=wl.num_q_heads, w_group=G, partition=1024)
    assert np.abs(q256 - qbig).max() <= 2e-4, "partition size changed the quantized result"
    assert np.abs(q256 - ref).max() <= 2e-2


def pin_decode_special_cases(orc, G=32):
    # (1) one token: output is the dequantized V of that token
    wl = tiny_decode(seed=12, seq_lens=(1, 1, 1))
    cache, q8, qs = orc.fill(wl)
    K, V, sK, sV = cache_rows(cache)
    out = orc.paged_decode(q8, qs, cache, wl.block_tables, wl.seq_lens,
                           num_q_heads=wl.num_q_heads, w_group=G)
    grp = wl.num_q_heads // wl.num_kv_heads
    for b in range(wl.num_seqs):
        sl = seq_slots(wl, b)
        for h in range(wl.num_q_heads):
            deq = np.float64(sV[sl[0], h // grp]) * V[sl[0], h // grp].astype(np.float64)
            assert np.all(np.abs(out[b, h] - deq) <= 4e-7 * np.abs(deq) + 1e-30), "L=1"
    # (2) equal scores (K = 0) and equal V scales: every Wq is 127, output is
    #     the mean of the dequantized V rows
    wl = tiny_decode(seed=13, seq_lens=(40, 600))
    wl.key[:] = 0
    rng = np.random.default_rng(13)
    base = np.clip(rng.standard_normal(wl.head_dim), -2.5, 2.5).astype(np.float32)
    base[0] = 3.0
    signs = rng.choice([-1.0, 1.0], size=wl.value.shape).astype(np.float32)
    wl.value[:] = W.f32_to_bf16_bits(signs * base[None, None, :])
    cache, q8, qs = orc.fill(wl)
    K, V, sK, sV = cache_rows(cache)
    out = orc.paged_decode(q8, qs, cache, wl.block_tables, wl.seq_lens,
                           num_q_heads=wl.num_q_heads, w_group=G)
    for b in range(wl.num_seqs):
        sl = seq_slots(wl, b)
        for h in range(wl.num_q_heads):
            kv = h // grp
            mean = (sV[sl, kv].astype(np.float64)[:, None] * V[sl, kv]).mean(0)
            assert np.all(np.abs(out[b, h] - mean) <= 1e-6 * (np.abs(mean) + 1e-2)), "equal scores"
    # (3) one dominant score: output is that token's dequantized V
    wl = tiny_decode(seed=14, seq_lens=(90,))
    qv = W.bf16_bits_to_f32(wl.query[0]).astype(np.float32)
    j = 37
    for h in range(wl.num_kv_heads):
        wl.key[j, h] = W.f32_to_bf16_bits(8.0 * qv[h * grp])
        wl.query[0, h * grp + 1:(h + 1) * grp] = wl.query[0, h * grp]
    cache, q8, qs = orc.fill(wl)
    K, V, sK, sV = cache_rows(cache)
    out = orc.paged_decode(q8, qs, cache, wl.block_tables, wl.seq_lens,
                           num_q_heads=wl.num_q_heads, w_group=G)
    sl = seq_slots(wl, 0)
    for h in range(wl.num_q_heads):
        kv = h // grp
        deq = np.float64(sV[sl[j], kv]) * V[sl[j], kv].astype(np.float64)
        assert np.abs(out[0, h] - deq).max() <= 1e-5 * np.abs(deq).max(), "dominant score"
    # (4) empty sequence writes zeros
    wl = tiny_decode(seed=15, seq_lens=(5, 3))
    cache, q8, qs = orc.fill(wl)
    out = orc.paged_decode(q8, qs, cache, wl.block_tables, np.array([0, 3], np.int32),
                           num_q_heads=wl.num_q_heads, w_group=G)
    assert not out[0].any()


# ---------------------------------------------------------------------------
# prefill
# ---------------------------------------------------------------------------
def _prefill_rows(wl):
    qsl = wl.query_start_loc
    res = []
    for b in range(wl.num_seqs):
        chunk = int(qsl[b + 1] - qsl[b])
        ctx = int(wl.seq_lens[b]) - chunk
        for j in range(chunk):
            res.append((int(qsl[b]) + j, b, ctx + j))
    return res


def pin_prefill_exact(orc, G=32, seed=9):
    """Exact online softmax over history + causal chunk equals plain softmax
    over the visible keys, for any tile size."""
    wl = tiny_prefill(seed=seed)
    cache, q8, qs = orc.fill(wl)
    K, V, sK, sV = cache_rows(cache)
    grp = wl.num_q_heads // wl.num_kv_heads
    ex = ORC_EXACT | ORC_NO_WQUANT
    args = (q8, qs, wl.query_start_loc, wl.seq_lens, cache, wl.block_tables)
    outs = [orc.prefix_prefill(*args, w_group=G, tile=t, flags=ex) for t in (256, 64, G)]
    ref = np.zeros_like(outs[0], dtype=np.float64)
    for r, b, pos in _prefill_rows(wl):
        sl = seq_slots(wl, b)[:pos + 1]
        for h in range(wl.num_q_heads):
            kv = h // grp
            acc = K[sl, kv].astype(np.int64) @ q8[r, h].astype(np.int64)
            s = acc * np.float64(qs[r, h]) * sK[sl, kv].astype(np.float64) * wl.softmax_scale
            p = _softmax64(s)
            ref[r, h] = (p * sV[sl, kv].astype(np.float64)) @ V[sl, kv].astype(np.float64)
    for o in outs:
        assert np.all(np.abs(o - ref) <= 1e-6 * (np.abs(ref) + 1e-3)), "exact prefill != softmax"


def pin_prefill_trace(orc, G=32, seed=10, tile=64):
    wl = tiny_prefill(seed=seed)
    cache, q8, qs = orc.fill(wl)
    K, V, sK, sV = cache_rows(cache)
    grp = wl.num_q_heads // wl.num_kv_heads
    rows = _prefill_rows(wl)
    ref = prefill_reference_fp64(wl)
    args = (q8, qs, wl.query_start_loc, wl.seq_lens, cache, wl.block_tables)
    for r, b, pos in rows[::3]:
        for h in range(0, wl.num_q_heads, 3):
            kv = h // grp
            tr = orc.prefill_row(*args, r, h, w_group=G, tile=tile)
            assert tr["nk"] == pos + 1
            sl = seq_slots(wl, b)[:pos + 1]
            acc = K[sl, kv].astype(np.int64) @ q8[r, h].astype(np.int64)
            s64 = acc * np.float64(qs[r, h]) * sK[sl, kv].astype(np.float64) * wl.softmax_scale
            assert np.all(np.abs(tr["s"] - s64) <= 2e-7 * np.abs(s64) + 1e-30), "score chain"
            nk = pos + 1
            mrun = -np.inf
            m_of = np.zeros(nk)
            for ti, t0 in enumerate(range(0, nk, tile)):
                t1 = min(nk, t0 + tile)
                mrun = max(mrun, float(tr["s"][t0:t1].max()))
                assert tr["m_tile"][ti] == np.float32(mrun), "running max"
                m_of[t0:t1] = mrun
            d = tr["s"].astype(np.float64) - m_of
            pt64 = np.exp(d)
            assert np.all(np.abs(tr["ptil"] - pt64) <= 1e-6 * (1 + np.abs(d)) * pt64 + 1e-45), "p~"
            Wt = (tr["ptil"] * sV[sl, kv]).astype(np.float32)
            for g0 in range(0, nk, G):
                g1 = min(nk, g0 + G)
                check_group_quant(Wt[g0:g1], tr["Wq"][g0:g1], tr["sW"][g0 // G],
                                  f"prefill row {r} head {h} group {g0 // G}")
            mf = m_of[-1]
            c_tok = np.exp(m_of - mf)
            sW_tok = np.repeat(tr["sW"].astype(np.float64), G)[:nk]
            o = (c_tok * sW_tok * tr["Wq"]) @ V[sl, kv].astype(np.float64)
            l = (c_tok * tr["ptil"]).sum()
            assert abs(tr["l"][0] - l) <= 1e-5 * l, "l = sum of unquantized p~"
            O = o / l
            assert np.all(np.abs(tr["out"] - O) <= 1e-5 * (np.abs(O) + 1e-3)), "o/l re-assembly"
            # a-priori bound against unquantized fp64 causal attention
            tok = np.nonzero(wl.token_seq == b)[0]
            tok = tok[np.argsort(wl.token_pos[tok])][:nk]
            Vorig = W.bf16_bits_to_f32(wl.value[tok, kv]).astype(np.float64)
            Korig = W.bf16_bits_to_f32(wl.key[tok, kv]).astype(np.float64)
            qorig = W.bf16_bits_to_f32(wl.query[r, h]).astype(np.float64)
            Pe = _softmax64(Korig @ qorig / np.sqrt(wl.head_dim))
            P = c_tok * tr["ptil"] / l
            bound = (np.abs(Pe - P) @ np.abs(Vorig)
                     + (P * sV[sl, kv] / 2).sum()
                     + (c_tok * sW_tok / l / 2 * (1 + 1e-6)) @ np.abs(V[sl, kv].astype(np.float64))
                     + 1e-5)
            assert np.all(np.abs(tr["out"] - ref[r, h]) <= bound), "prefill error above bound"


def pin_prefill_bf16_pv(orc, seed=17, tile=64):
    """The prefill BF16-PV ablation: scores, running maxima, p~ and l equal
    the int8 path's; W = bf16(p~ * sV) as torch rounds it; the output equals
    the re-assembly sum c_tok W Vq / l and stays within the bound against
    fp64 causal attention with the bf16 term 2^-9 P sV |Vq|."""
    import torch
    from oracle import ORC_BF16_PV
    wl = tiny_prefill(seed=seed)
    cache, q8, qs = orc.fill(wl)
    K, V, sK, sV = cache_rows(cache)
    grp = wl.num_q_heads // wl.num_kv_heads
    ref = prefill_reference_fp64(wl)
    args = (q8, qs, wl.query_start_loc, wl.seq_lens, cache, wl.block_tables)
    for r, b, pos in _prefill_rows(wl)[::4]:
        for h in range(0, wl.num_q_heads, 3):
            kv = h // grp
            tb = orc.prefill_row(*args, r, h, tile=tile, flags=ORC_BF16_PV)
            t8 = orc.prefill_row(*args, r, h, tile=tile)
            for k in ("s", "ptil", "m_tile", "l"):
                assert np.array_equal(tb[k], t8[k]), f"bf16-PV prefill changed {k}"
            nk = pos + 1
            sl = seq_slots(wl, b)[:nk]
            w32 = (tb["ptil"] * sV[sl, kv]).astype(np.float32)
            wb = torch.from_numpy(w32).to(torch.bfloat16).to(torch.float32).numpy().astype(np.float64)
            m_of = np.zeros(nk)
            mrun = -np.inf
            for ti, t0 in enumerate(range(0, nk, tile)):
                mrun = float(tb["m_tile"][ti])
                m_of[t0:t0 + tile] = mrun
            c_tok = np.exp(m_of - m_of[-1])
            vq = V[sl, kv].astype(np.float64)
            O = (c_tok * wb) @ vq / tb["l"][0]
            assert np.all(np.abs(tb["out"] - O) <= 1e-5 * (np.abs(O) + 1e-3)), "o/l re-assembly"
            tok = np.nonzero(wl.token_seq == b)[0]
            tok = tok[np.argsort(wl.token_pos[tok])][:nk]
            Vorig = W.bf16_bits_to_f32(wl.value[tok, kv]).astype(np.float64)
            Korig = W.bf16_bits_to_f32(wl.key[tok, kv]).astype(np.float64)
            qorig = W.bf16_bits_to_f32(wl.query[r, h]).astype(np.float64)
            Pe = _softmax64(Korig @ qorig / np.sqrt(wl.head_dim))
            P = c_tok * tb["ptil"] / tb["l"][0]
            sVt = sV[sl, kv].astype(np.float64)
            bound = (np.abs(Pe - P) @ np.abs(Vorig) + (P * sVt / 2).sum()
                     + (2.0 ** -9 * P * sVt * (1 + 1e-6)) @ np.abs(vq) + 1e-5)
            assert np.all(np.abs(tb["out"] - ref[r, h]) <= bound), "bf16-PV prefill above bound"


def pin_prefill_uint8_w(orc, G=32, seed=20, tile=64):
    """The UINT8-W prefill (the PV-MMAC page's section 6 candidate in the
    prefill's online softmax): scores, running maxima, p~ and l equal the int8
    path's; per aligned group sW = max W / 255 bit for bit and Wq the
    brute-force nearest codes of W / sW over 0..255; the output equals the
    re-assembly sum c_tok sW Wq Vq / l and stays within the bound against fp64
    causal attention with the sW / 2 term; on average it is closer to fp64
    attention than int8 W."""
    from oracle import ORC_UINT8_W
    wl = tiny_prefill(seed=seed)
    cache, q8, qs = orc.fill(wl)
    K, V, sK, sV = cache_rows(cache)
    grp = wl.num_q_heads // wl.num_kv_heads
    ref = prefill_reference_fp64(wl)
    args = (q8, qs, wl.query_start_loc, wl.seq_lens, cache, wl.block_tables)
    err_u = err8 = 0.0
    for r, b, pos in _prefill_rows(wl)[::3]:
        for h in range(0, wl.num_q_heads, 2):
            kv = h // grp
            tu = orc.prefill_row(*args, r, h, w_group=G, tile=tile, flags=ORC_UINT8_W)
            t8 = orc.prefill_row(*args, r, h, w_group=G, tile=tile)
            for k in ("s", "ptil", "m_tile", "l"):
                assert np.array_equal(tu[k], t8[k]), f"uint8-W prefill changed {k}"
            nk = pos + 1
            sl = seq_slots(wl, b)[:nk]
            w32 = (tu["ptil"] * sV[sl, kv]).astype(np.float32)
            wq = tu["Wq"].view(np.uint8).astype(np.int64)
            for g0 in range(0, nk, G):
                g1 = min(nk, g0 + G)
                w = w32[g0:g1]
                sw = tu["sW"][g0 // G]
                exp_sw = np.float32(w.max()) / np.float32(255) if w.max() > 0 else np.float32(0)
                assert sw.view(np.uint32) == np.float32(exp_sw).view(np.uint32), "group sW"
                if sw > 0:
                    assert np.array_equal(wq[g0:g1], nearest_code_u8((w / sw).astype(np.float32))), \
                        "group codes"
                else:
                    assert not wq[g0:g1].any()
            m_of = np.zeros(nk)
            for ti, t0 in enumerate(range(0, nk, tile)):
                m_of[t0:min(nk, t0 + tile)] = float(tu["m_tile"][ti])
            c_tok = np.exp(m_of - m_of[-1])
            sW_tok = np.repeat(tu["sW"].astype(np.float64), G)[:nk]
            vq = V[sl, kv].astype(np.float64)
            o = (c_tok * sW_tok * wq) @ vq
            l = float(tu["l"][0])
            assert np.all(np.abs(tu["out"] - o / l) <= 1e-5 * (np.abs(o / l) + 1e-3)), \
                "o/l re-assembly"
            tok = np.nonzero(wl.token_seq == b)[0]
            tok = tok[np.argsort(wl.token_pos[tok])][:nk]
            Vorig = W.bf16_bits_to_f32(wl.value[tok, kv]).astype(np.float64)
            Korig = W.bf16_bits_to_f32(wl.key[tok, kv]).astype(np.float64)
            qorig = W.bf16_bits_to_f32(wl.query[r, h]).astype(np.float64)
            Pe = _softmax64(Korig @ qorig / np.sqrt(wl.head_dim))
            P = c_tok * tu["ptil"] / l
            bound = (np.abs(Pe - P) @ np.abs(Vorig) + (P * sV[sl, kv] / 2).sum()
                     + (c_tok * sW_tok / l / 2 * (1 + 1e-6)) @ np.abs(vq) + 1e-5)
            assert np.all(np.abs(tu["out"] - ref[r, h]) <= bound), "uint8-W prefill above bound"
            err_u += np.abs(tu["out"] - ref[r, h]).mean()
            err8 += np.abs(t8["out"] - ref[r, h]).mean()
    assert err_u < err8, f"uint8 W not more accurate on average ({err_u} vs {err8})"


def pin_prefill_vs_decode(orc, G=32, seed=9):
    """A prefill row equals a decode of the same query over its visible keys
    (exactly in real arithmetic; here up to fp32 rounding)."""
    wl = tiny_prefill(seed=seed)
    cache, q8, qs = orc.fill(wl)
    out = orc.prefix_prefill(q8, qs, wl.query_start_loc, wl.seq_lens, cache,
                             wl.block_tables, w_group=G)
    worst = 0.0
    for r, b, pos in _prefill_rows(wl):
        d = orc.paged_decode(q8[r][None], qs[r][None], cache, wl.block_tables[b][None],
                             np.array([pos + 1], np.int32), num_q_heads=wl.num_q_heads,
                             w_group=G)
        worst = max(worst, float(np.abs(d[0] - out[r]).max()))
    assert worst <= 2e-4, f"prefill row differs from decode by {worst}"
    return worst


def _q_bf16_from_codes(q8, shift=6):
    """bf16 bits of q8 * 2^-shift: exact, since |q8| <= 127 needs 7 bits."""
    return W.f32_to_bf16_bits(q8.astype(np.float32) * np.float32(2.0 ** -shift))


def pin_decode_bf16_qk(orc, G=32, seed=18):
    """The BF16-QK ablation (decode).
    (1) A bf16 query equal to int8 codes times 2^-6 must give, bit for bit,
        the int8 path's output with q_scale = 2^-6 (the dot product is then
        acc * sQ exactly, and the rest is shared).
    (2) Exact mode: softmax attention of the bf16 query over the dequantized
        cache, written here with numpy in fp64.
    (3) With the W groups, one partition: within the a-priori bound against
        unquantized fp64 attention -- the QK term from the bf16 query's own
        probabilities (no Q quantization), plus |eV| <= sV/2 and
        |eW| <= sW/2 with sW = max P sV / 127 per group."""
    wl = tiny_decode(seed=seed, seq_lens=(1, 9, 40, 256, 300, 600))
    cache, q8, qs = orc.fill(wl)
    K, V, sK, sV = cache_rows(cache)
    grp = wl.num_q_heads // wl.num_kv_heads
    tables = (cache, wl.block_tables, wl.seq_lens)
    # (1)
    qb = _q_bf16_from_codes(q8)
    for flags in (0, ORC_NO_WQUANT):
        o8 = orc.paged_decode(q8, np.full_like(qs, 2.0 ** -6), *tables,
                              num_q_heads=wl.num_q_heads, w_group=G, flags=flags)
        ob = orc.paged_decode_bf16qk(qb, *tables, w_group=G, flags=flags)
        assert np.array_equal(o8, ob), "bf16-QK with q = codes * 2^-6 != int8 path"
    # (2) and (3): the workload's own bf16 queries
    qrows = wl.decode_query_rows()
    qreal = wl.query[qrows]
    ex = orc.paged_decode_bf16qk(qreal, *tables, w_group=G, flags=ORC_EXACT | ORC_NO_WQUANT)
    ref = decode_reference_fp64(wl)
    for b in range(wl.num_seqs):
        L = int(wl.seq_lens[b])
        sl = seq_slots(wl, b)
        big = 256 * -(-L // 256)
        ob = orc.paged_decode_bf16qk(qreal[b:b + 1], cache, wl.block_tables[b:b + 1],
                                     wl.seq_lens[b:b + 1], w_group=G, partition=big)[0]
        tok = np.nonzero(wl.token_seq == b)[0]
        tok = tok[np.argsort(wl.token_pos[tok])]
        for h in range(wl.num_q_heads):
            kv = h // grp
            qf = W.bf16_bits_to_f32(qreal[b, h]).astype(np.float64)
            kdq = K[sl, kv].astype(np.float64) * sK[sl, kv].astype(np.float64)[:, None]
            sVt = sV[sl, kv].astype(np.float64)
            vq = V[sl, kv].astype(np.float64)
            p = _softmax64(kdq @ qf * wl.softmax_scale)
            want = (p * sVt) @ vq
            assert np.all(np.abs(ex[b, h] - want) <= 1e-6 * (np.abs(want) + 1e-3)), \
                f"exact bf16-QK decode seq {b} head {h} != softmax over the dequantized cache"
            Vorig = W.bf16_bits_to_f32(wl.value[tok, kv]).astype(np.float64)
            Korig = W.bf16_bits_to_f32(wl.key[tok, kv]).astype(np.float64)
            Pe = _softmax64(Korig @ qf / np.sqrt(wl.head_dim))
            wmax = np.array([(p[g:g + G] * sVt[g:g + G]).max() for g in range(0, L, G)])
            sWt = np.repeat(wmax / 127 * (1 + 1e-5), G)[:L]
            bound = (np.abs(Pe - p) @ np.abs(Vorig) + (p * sVt / 2).sum()
                     + (sWt / 2) @ np.abs(vq)) * (1 + 1e-4) + 1e-6
            err = np.abs(ob[h] - ref[b, h])
            assert np.all(err <= bound), f"bf16-QK decode seq {b} head {h}: error above bound"


def pin_prefill_bf16_qk(orc, G=32, seed=19):
    """The BF16-QK ablation (prefill): (1) bit for bit the int8 path when the
    bf16 query is int8 codes times 2^-6 and q_scale = 2^-6, for two tile
    sizes; (2) exact mode equals causal softmax attention of the bf16 query
    over the dequantized cache, written here with numpy in fp64."""
    wl = tiny_prefill(seed=seed)
    cache, q8, qs = orc.fill(wl)
    K, V, sK, sV = cache_rows(cache)
    grp = wl.num_q_heads // wl.num_kv_heads
    loc = (wl.query_start_loc, wl.seq_lens, cache, wl.block_tables)
    qb = _q_bf16_from_codes(q8)
    for tile in (256, 64):
        o8 = orc.prefix_prefill(q8, np.full_like(qs, 2.0 ** -6), *loc, w_group=G, tile=tile)
        ob = orc.prefix_prefill_bf16qk(qb, *loc, w_group=G, tile=tile)
        assert np.array_equal(o8, ob), "bf16-QK prefill with q = codes * 2^-6 != int8 path"
    qreal = wl.query  # [Tq, Hq, D]: the chunk's bf16 queries, row for row
    ex = orc.prefix_prefill_bf16qk(qreal, *loc, w_group=G, tile=64,
                                   flags=ORC_EXACT | ORC_NO_WQUANT)
    for r, b, pos in _prefill_rows(wl):
        sl = seq_slots(wl, b)[:pos + 1]
        for h in range(wl.num_q_heads):
            kv = h // grp
            qf = W.bf16_bits_to_f32(qreal[r, h]).astype(np.float64)
            kdq = K[sl, kv].astype(np.float64) * sK[sl, kv].astype(np.float64)[:, None]
            p = _softmax64(kdq @ qf * wl.softmax_scale)
            want = (p * sV[sl, kv].astype(np.float64)) @ V[sl, kv].astype(np.float64)
            assert np.all(np.abs(ex[r, h] - want) <= 1e-6 * (np.abs(want) + 1e-3)), \
                f"exact bf16-QK prefill row {r} head {h} != causal softmax"


ALL_PINS = [pin_quantize_golden, pin_quantize_bruteforce, pin_cache_layout,
            pin_decode_trace, pin_decode_bruteforce, pin_decode_partition_invariance,
            pin_decode_special_cases, pin_prefill_exact, pin_prefill_trace,
            pin_prefill_vs_decode, pin_rope_rotation, pin_rope_producer,
            pin_bf16_rounding, pin_decode_bf16_pv, pin_quantize_w_u8, pin_decode_uint8_w,
            pin_decode_multi_query, pin_prefill_bf16_pv, pin_decode_bf16_qk,
            pin_prefill_bf16_qk, pin_prefill_uint8_w]
