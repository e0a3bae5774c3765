"""Mutation tests for the oracle's pins (CPU only).

Each case plants one plausible mistake in a copy of oracle/oracle.cpp (a text
patch; the shipped oracle has no planted code paths), builds the copy with the
same flags, and requires at least one pin of tests/pins.py to fail.  This is
what shows that the pins would catch a dropped term, a wrong sign or index, a
transposed operand, a wrong rounding rule or a mis-grouped scale -- the last
one is the negative control the PV-MMAC page describes in section 4 (scales
computed on tokens other than the ones a matrix instruction consumes).
"""
from __future__ import annotations

import sys
from pathlib import Path

import pytest

import pins

ROOT = Path(__file__).resolve().parent.parent
SRC = ROOT / "oracle" / "oracle.cpp"

# name -> list of (original text, replacement); every original must occur.
MUTANTS = {
    "round_half_even": [("float r = std::round(x[i] / s);",
                         "float r = std::nearbyint(x[i] / s);")],
    "round_truncate": [("float r = std::round(x[i] / s);",
                        "float r = std::trunc(x[i] / s);")],
    "scale_over_128": [("const float s = amax / 127.0f;", "const float s = amax / 128.0f;")],
    "gqa_modulo": [("head / (Hq / Hkv)}", "head % Hkv}")],
    "k_layout_token_major": [
        ("((((size_t)blk * Hkv + h) * (D / 16) + d / 16) * bs + off) * 16 + d % 16",
         "((((size_t)blk * Hkv + h) * bs + off) * (D / 16) + d / 16) * 16 + d % 16")],
    "v_layout_dim_inner": [("(((size_t)blk * Hkv + h) * D + d) * bs + off",
                            "(((size_t)blk * Hkv + h) * bs + off) * D + d")],
    "scale_layout_head_major": [("((size_t)blk * bs + off) * Hkv + h",
                                 "((size_t)blk * Hkv + h) * bs + off")],
    "page_offset_shift": [("int off(int i) const { return i % c->bs; }",
                           "int off(int i) const { return (i + 1) % c->bs; }")],
    "k_unsigned": [("acc += (int64_t)q[d] * (int64_t)sv.kq(i, d);",
                    "acc += (int64_t)q[d] * (int64_t)(uint8_t)sv.kq(i, d);")],
    "score_drops_sk": [("  s = s * sk;\n", "  s = s * 1.0f;\n  (void)sk;\n")],
    "v_scale_reads_k_scale": [("float sv(int i) const { return c->vs[",
                               "float sv(int i) const { return c->ks[")],
    "decode_w_without_vscale": [("W[i] = P[i] * sv.sv(i0 + i);", "W[i] = P[i];")],
    "prefill_w_without_vscale": [("W[j] = pt[j] * sv.sv(t0 + j);", "W[j] = pt[j];")],
    "decode_p_unnormalized": [("P[i] = e[i] / l;", "P[i] = e[i];")],
    "exp_base_two": [("return (float)std::exp((double)x);", "return (float)std::exp2((double)x);")],
    "merge_without_exp": [("const double w = l_part[p] * std::exp(m_part[p] - M);",
                           "const double w = l_part[p];")],
    "merge_without_l": [("const double w = l_part[p] * std::exp(m_part[p] - M);",
                         "const double w = std::exp(m_part[p] - M);")],
    "misgrouped_w_scale": [(
        "orc_quantize_w(W, n, wq.data(), &sw);",
        "orc_quantize_w(W, (n + 1) / 2, wq.data(), &sw);\n"
        "  for (int j = 0; j < n; ++j)\n"
        "    wq[j] = sw > 0 ? (int8_t)std::min(127.0f, std::round(W[j] / sw)) : 0;")],
    "prefill_no_alpha": [("for (int d = 0; d < D; ++d) o[d] *= (double)alpha;", "")],
    "prefill_l_of_w": [("psum += (double)pt[j];", "psum += (double)pt[j] * sv.sv(t0 + j);")],
    "prefill_not_causal": [("const int pos = ctx + (row - query_start_loc[b]);",
                            "const int pos = seq_lens[b] - 1;")],
    "prefill_excludes_self": [("const int nk = pos + 1;", "const int nk = pos > 0 ? pos : 1;")],
    "u8_scale_127": [("  const float s = amax / 255.0f;", "  const float s = amax / 127.0f;")],
    "u8_clamp_127": [("    if (r > 255.0f) r = 255.0f;", "    if (r > 127.0f) r = 127.0f;")],
    "u8_round_down": [("    float r = std::round(w[i] / s);\n    if (r > 255.0f)",
                       "    float r = std::floor(w[i] / s);\n    if (r > 255.0f)")],
    "u8_flag_ignored": [("      if (quant_w && u8_w) {\n        add_group_quantized_u8(&W[g0], i0 + g0",
                         "      if (false) {\n        add_group_quantized_u8(&W[g0], i0 + g0")],
    "prefill_u8_flag_ignored": [("      if (quant_w && u8_w) {\n        /* [PV 6]",
                                 "      if (false) {\n        /* [PV 6]")],
    "prefill_bf16_ignored": [("      if (bf16_pv) W[j] = round_to_bf16(W[j]);", "")],
    "prefill_bf16_before_sv": [("      if (bf16_pv) W[j] = round_to_bf16(W[j]);",
                                "      if (bf16_pv) W[j] = round_to_bf16(pt[j]) * sv.sv(t0 + j);")],
    "bf16_truncates": [("  u += 0x7fffu + ((u >> 16) & 1u);\n", "")],
    "bf16_ties_up": [("  u += 0x7fffu + ((u >> 16) & 1u);", "  u += 0x8000u;")],
    "bf16_before_sv": [("      if (bf16_pv) W[i] = round_to_bf16(W[i]);",
                        "      if (bf16_pv) W[i] = round_to_bf16(P[i]) * sv.sv(i0 + i);")],
    "bf16_pv_ignored": [("      if (bf16_pv) W[i] = round_to_bf16(W[i]);", "")],
    "rope_inverse_turn": [("    x[j] = a - b;\n    x[j + h] = e + f;",
                           "    x[j] = a + b;\n    x[j + h] = e - f;")],
    "rope_cos_sin_swapped": [("c = cs[j], s = cs[h + j];", "c = cs[h + j], s = cs[j];")],
    "rope_interleaved_pairs": [(
        "    const float x1 = x[j], x2 = x[j + h], c = cs[j], s = cs[h + j];\n"
        "    const float a = x1 * c, b = x2 * s, e = x2 * c, f = x1 * s;\n"
        "    x[j] = a - b;\n"
        "    x[j + h] = e + f;",
        "    const float x1 = x[2 * j], x2 = x[2 * j + 1], c = cs[j], s = cs[h + j];\n"
        "    const float a = x1 * c, b = x2 * s, e = x2 * c, f = x1 * s;\n"
        "    x[2 * j] = a - b;\n"
        "    x[2 * j + 1] = e + f;")],
    "rope_half_dims": [("  const int h = R / 2;\n  for (int j = 0; j < h; ++j) {",
                        "  const int h = R / 2;\n  for (int j = 0; j < h / 2; ++j) {")],
    "rope_skips_query": [("x[d] = bf16_to_float(src[d]);\n        if (cs) rope_rotate(x.data(), R, cs);",
                          "x[d] = bf16_to_float(src[d]);")],
    "rope_rotates_value": [("x[d] = bf16_to_float(vs[d]);\n",
                            "x[d] = bf16_to_float(vs[d]);\n      if (cs) rope_rotate(x.data(), R, cs);\n")],
    "rope_position_off_by_one": [("cos_sin + (size_t)positions[t] * R",
                                  "cos_sin + (size_t)(positions[t] > 0 ? positions[t] - 1 : 1) * R")],
    "bf16qk_k_unsigned": [("acc += (double)bf16_to_float(q[d]) * (double)sv.kq(i, d);",
                           "acc += (double)bf16_to_float(q[d]) * (double)(uint8_t)sv.kq(i, d);")],
    "bf16qk_query_truncated": [("acc += (double)bf16_to_float(q[d]) * (double)sv.kq(i, d);",
                                "acc += (double)(int)bf16_to_float(q[d]) * (double)sv.kq(i, d);")],
    "bf16qk_dims_reversed": [("acc += (double)bf16_to_float(q[d]) * (double)sv.kq(i, d);",
                              "acc += (double)bf16_to_float(q[D - 1 - d]) * (double)sv.kq(i, d);")],
    "bf16qk_first_head_query": [("Query{nullptr, 0.0f, q_bf16 + qr * D}",
                                 "Query{nullptr, 0.0f, q_bf16 + qr / Hq * Hq * D}")],
    "bf16qk_score_drops_sk": [("  float s = (float)dot;\n  s = s * sk;\n",
                               "  float s = (float)dot;\n  (void)sk;\n")],
    "bf16qk_exact_drops_sk": [("*s64 = dot * (double)sv.sk(i) * (double)softmax_scale;",
                               "*s64 = dot * (double)softmax_scale;")],
    "rope_after_quantize": [(
        "      if (cs) rope_rotate(x.data(), R, cs);\n      orc_quantize(x.data(), D, q.data(), &s);\n"
        "      for (int d = 0; d < D; ++d) k_cache",
        "      orc_quantize(x.data(), D, q.data(), &s);\n"
        "      if (cs) { for (int d = 0; d < D; ++d) x[d] = q[d]; rope_rotate(x.data(), R, cs);\n"
        "        for (int d = 0; d < D; ++d) q[d] = (int8_t)std::max(-127.0f, std::min(127.0f, std::round(x[d]))); }\n"
        "      for (int d = 0; d < D; ++d) k_cache")],
}


def build_mutant(name: str, tmp_path: Path):
    sys.path.insert(0, str(ROOT))
    from oracle import Oracle, build as obuild
    src = SRC.read_text()
    for old, new in MUTANTS[name]:
        assert src.count(old) >= 1, f"mutation {name}: pattern not found"
        src = src.replace(old, new)
    d = tmp_path / name
    d.mkdir()
    (d / "oracle.cpp").write_text(src)
    lib = obuild.build(d / "oracle.cpp", d / "liboracle.so", extra=["-w"])
    return Oracle(lib)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    orc = build_mutant(name, tmp_path)
    failed = []
    for pin in pins.ALL_PINS:
        try:
            pin(orc)
        except AssertionError as e:
            failed.append((pin.__name__, str(e).splitlines()[0] if str(e) else ""))
        except (ValueError, FloatingPointError, IndexError) as e:
            failed.append((pin.__name__, repr(e)))
    assert failed, f"no pin caught the planted mistake {name!r}"
    print(f"{name}: caught by {[f[0] for f in failed]}")


def test_misgrouped_scale_blows_past_bound(tmp_path):
    """Negative control (PV-MMAC page, section 4): scales taken from tokens other
    than the ones the group consumes push the decode error far past the
    a-priori bound that the correct grouping satisfies."""
    import numpy as np
    import oracle as O
    import workloads as W
    from refmath import decode_reference_fp64
    good = O.default()
    bad = build_mutant("misgrouped_w_scale", tmp_path)
    wl = pins.tiny_decode(seed=31, seq_lens=(200, 256))
    ref = decode_reference_fp64(wl)
    errs = []
    for orc in (good, bad):
        cache, q8, qs = orc.fill(wl)
        out = orc.paged_decode(q8, qs, cache, wl.block_tables, wl.seq_lens,
                               num_q_heads=wl.num_q_heads)
        errs.append(float(np.abs(out - ref).max()))
    print(f"max-abs vs fp64: grouped {errs[0]:.3g}, mis-grouped {errs[1]:.3g}")
    assert errs[1] > 10 * errs[0]
