/*
 * CPU oracle for paged attention over an INT8 KV cache -- TEST INFRASTRUCTURE.
 *
 * Plain, slow and single-threaded on purpose: every loop follows the pages'
 * formulas in their order, with no blocking or fusion beyond what they state.
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg use it.
 * It shares nothing with the HIP library.
 *
 * Pages (by title):
 *  [KV] "INT8 KV and INT8 MMAC attention inference optimisation on a gfx936 DCU"
 *  [PV] "Implementing INT8 PV MMAC on a gfx936 DCU: V-scale fusion,
 *       probability quantization, fragment grouping"
 *
 * Readings of points the pages leave open (each is listed in the design notes):
 *  - rounding is half away from zero (std::round) for K, V, Q and W;
 *  - amax == 0 stores scale 0 and all-zero codes;
 *  - the exponential of an fp32 argument is the correctly rounded fp32 e^x;
 *  - a W group is an aligned, contiguous block of G absolute token positions;
 *    groups never straddle a decode partition or a prefill key tile;
 *  - q head h reads KV head h / (Hq / Hkv);
 *  - the score is ((acc * sQ) * sK) * softmax_scale, left to right in fp32;
 *  - partitions are merged with weights l_p * exp(m_p - M), M = max m_p.
 *  - RoPE, where the producer applies it, is the rotate-half pairing over
 *    the first R dims with a caller-given cos|sin table per position, each
 *    product and the sum / difference rounded to fp32; V is not rotated.
 *
 * Parity pins: see the oracle tests (worked quantization example, brute force
 * against unquantized fp64 attention with an a-priori bound, partition/tile
 * invariance, the error decomposition, ranges, special cases, layout
 * re-derivation).  No function here is left unpinned.
 */
#include "oracle.h"

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <limits>
#include <vector>

namespace {

float bf16_to_float(uint16_t b) {
  uint32_t u = static_cast<uint32_t>(b) << 16;
  float f;
  std::memcpy(&f, &u, sizeof f);
  return f;
}

/* Cache geometry and addressing [KV 2.3]:
 *   K [nb, Hkv, D/16, bs, 16]: 16 head-dim bytes contiguous per token,
 *   V [nb, Hkv, D, bs]:        tokens innermost,
 *   scales [nb, bs, Hkv] fp32. */
struct Cache {
  int Hq, Hkv, D, bs, nb;
  const int8_t* k;
  const int8_t* v;
  const float* ks;
  const float* vs;

  size_t k_index(int blk, int h, int off, int d) const {
    return ((((size_t)blk * Hkv + h) * (D / 16) + d / 16) * bs + off) * 16 + d % 16;
  }
  size_t v_index(int blk, int h, int off, int d) const {
    return (((size_t)blk * Hkv + h) * D + d) * bs + off;
  }
  size_t s_index(int blk, int h, int off) const {
    return ((size_t)blk * bs + off) * Hkv + h;
  }
};

/* Token i of a sequence lives in page table[i / bs] at offset i % bs. */
struct SeqView {
  const Cache* c;
  const int32_t* table;
  int kv;
  int page(int i) const { return table[i / c->bs]; }
  int off(int i) const { return i % c->bs; }
  int8_t kq(int i, int d) const { return c->k[c->k_index(page(i), kv, off(i), d)]; }
  int8_t vq(int i, int d) const { return c->v[c->v_index(page(i), kv, off(i), d)]; }
  float sk(int i) const { return c->ks[c->s_index(page(i), kv, off(i))]; }
  float sv(int i) const { return c->vs[c->s_index(page(i), kv, off(i))]; }
};

/* int32 QK accumulator: exact integer dot product of the int8 query and the
 * int8 key [PV 2; KV 3.3]. */
int32_t qk_acc(const int8_t* q, const SeqView& sv, int i, int D) {
  int64_t acc = 0;
  for (int d = 0; d < D; ++d) acc += (int64_t)q[d] * (int64_t)sv.kq(i, d);
  return (int32_t)acc;
}

/* Score recovery [PV 2]: score = acc * sQ * sK / sqrt(d), in fp32, multiplied
 * left to right. */
float score_f32(int32_t acc, float sq, float sk, float softmax_scale) {
  float s = (float)acc * sq;
  s = s * sk;
  s = s * softmax_scale;
  return s;
}

double score_f64(int32_t acc, float sq, float sk, float softmax_scale) {
  return (double)acc * (double)sq * (double)sk * (double)softmax_scale;
}

/* BF16-QK ablation (the QK row of the operator-level comparison [KV 4.1];
 * [PV 5] switches the PV half): the query is not quantized
 * and its bf16 values meet the int8 K codes exactly.  Each product has at
 * most 16 significant bits, the sum over d is taken in fp64 and rounded once
 * to fp32, and the score is (dot * sK) * softmax_scale in fp32, the int8
 * path's formula with acc * sQ replaced by the dot product. */
double qk_dot_bf16(const uint16_t* q, const SeqView& sv, int i, int D) {
  double acc = 0.0;
  for (int d = 0; d < D; ++d) acc += (double)bf16_to_float(q[d]) * (double)sv.kq(i, d);
  return acc;
}

float score_bf16qk_f32(double dot, float sk, float softmax_scale) {
  float s = (float)dot;
  s = s * sk;
  s = s * softmax_scale;
  return s;
}

/* The query of one (row, q head): int8 codes and their scale, or (BF16-QK)
 * the bf16 values. */
struct Query {
  const int8_t* q8;
  float sq;
  const uint16_t* q16;

  void score(const SeqView& sv, int i, int D, float softmax_scale, float* s, double* s64,
             int32_t* acc) const {
    if (q16) {
      const double dot = qk_dot_bf16(q16, sv, i, D);
      *s = score_bf16qk_f32(dot, sv.sk(i), softmax_scale);
      *s64 = dot * (double)sv.sk(i) * (double)softmax_scale;
      *acc = 0;
      return;
    }
    *acc = qk_acc(q8, sv, i, D);
    *s = score_f32(*acc, sq, sv.sk(i), softmax_scale);
    *s64 = score_f64(*acc, sq, sv.sk(i), softmax_scale);
  }
};

/* Contribution of one W group to the output [PV 1, 3]:
 *   c[d] = sW * sum_{i in group} Wq_i * Vq_i[d]   (inner sum exact integer). */
void add_group_quantized(const float* W, int i0, int n, const SeqView& sv, int D,
                         double weight, double* o, int8_t* wq_out, float* sw_out) {
  std::vector<int8_t> wq(n);
  float sw = 0.0f;
  orc_quantize_w(W, n, wq.data(), &sw);
  if (wq_out) std::memcpy(wq_out, wq.data(), n);
  if (sw_out) *sw_out = sw;
  for (int d = 0; d < D; ++d) {
    int64_t acc = 0;
    for (int j = 0; j < n; ++j) acc += (int64_t)wq[j] * (int64_t)sv.vq(i0 + j, d);
    o[d] += weight * (double)sw * (double)acc;
  }
}

/* The UINT8-W variant of one group: sW = max W / 255, Wq = round(W / sW) in
 * [0, 255], c[d] = sW * sum Wq_i * Vq_i[d] (exact integer inner sum). */
void add_group_quantized_u8(const float* W, int i0, int n, const SeqView& sv, int D,
                            double weight, double* o, int8_t* wq_out, float* sw_out) {
  std::vector<uint8_t> wq(n);
  float sw = 0.0f;
  orc_quantize_w_u8(W, n, wq.data(), &sw);
  if (wq_out) std::memcpy(wq_out, wq.data(), n);
  if (sw_out) *sw_out = sw;
  for (int d = 0; d < D; ++d) {
    int64_t acc = 0;
    for (int j = 0; j < n; ++j) acc += (int64_t)wq[j] * (int64_t)sv.vq(i0 + j, d);
    o[d] += weight * (double)sw * (double)acc;
  }
}

/* Unquantized W: c[d] = sum_i W_i * Vq_i[d] (used by the invariance pins). */
template <typename T>
void add_group_plain(const T* W, int i0, int n, const SeqView& sv, int D,
                     double weight, double* o) {
  for (int d = 0; d < D; ++d) {
    double acc = 0.0;
    for (int j = 0; j < n; ++j) acc += (double)W[j] * (double)sv.vq(i0 + j, d);
    o[d] += weight * acc;
  }
}

/* fp32 -> bf16 -> fp32 with round-to-nearest-even on the dropped 16 bits
 * (finite inputs). */
float round_to_bf16(float x) {
  uint32_t u;
  std::memcpy(&u, &x, 4);
  u += 0x7fffu + ((u >> 16) & 1u);
  u &= 0xffff0000u;
  float r;
  std::memcpy(&r, &u, 4);
  return r;
}

bool geometry_ok(int Hq, int Hkv, int D, int bs, int nb) {
  return Hq > 0 && Hkv > 0 && Hq % Hkv == 0 && D > 0 && D % 16 == 0 && bs > 0 &&
         nb >= 0;
}

}  // namespace

extern "C" {

float orc_expf(float x) { return (float)std::exp((double)x); }

/* [KV 2.1] amax = max|x|; scale = amax / 127; q = clamp(round(x/scale), ±127). */
void orc_quantize(const float* x, int n, int8_t* q, float* scale) {
  float amax = 0.0f;
  for (int i = 0; i < n; ++i) amax = std::max(amax, std::fabs(x[i]));
  if (amax == 0.0f) {
    *scale = 0.0f;
    for (int i = 0; i < n; ++i) q[i] = 0;
    return;
  }
  const float s = amax / 127.0f;
  *scale = s;
  for (int i = 0; i < n; ++i) {
    float r = std::round(x[i] / s);
    if (r > 127.0f) r = 127.0f;
    if (r < -127.0f) r = -127.0f;
    q[i] = (int8_t)r;
  }
}

/* UINT8 W ([PV] 6 names it as the candidate with one more bit, since W >= 0):
 * sW = max W / 255, Wq = round(W / sW) in [0, 255], ties away from zero;
 * max W == 0 gives sW = 0 and Wq = 0. */
void orc_quantize_w_u8(const float* w, int n, uint8_t* wq, float* sw) {
  float amax = 0.0f;
  for (int i = 0; i < n; ++i) amax = std::max(amax, std::fabs(w[i]));
  if (amax == 0.0f) {
    *sw = 0.0f;
    for (int i = 0; i < n; ++i) wq[i] = 0;
    return;
  }
  const float s = amax / 255.0f;
  *sw = s;
  for (int i = 0; i < n; ++i) {
    float r = std::round(w[i] / s);
    if (r > 255.0f) r = 255.0f;
    if (r < 0.0f) r = 0.0f;
    wq[i] = (uint8_t)r;
  }
}

/* [PV 1] sW = max(|W_group|) / 127, Wq = round(W / sW): the same symmetric
 * rule applied to the (non-negative) weights of one group. */
void orc_quantize_w(const float* w, int n, int8_t* wq, float* sw) {
  orc_quantize(w, n, wq, sw);
}

/* [KV 2.2] step 2, in the reading documented in oracle.h: the rotate-half
 * pairing (j, j + R/2) for j < R/2, turned by the tabulated cosine / sine of
 * the token's position; each product and the difference / sum rounded to
 * fp32 on its own (no fused multiply-add). */
static void rope_rotate(float* x, int R, const float* cs /* [R]: cos, then sin */) {
  const int h = R / 2;
  for (int j = 0; j < h; ++j) {
    const float x1 = x[j], x2 = x[j + h], c = cs[j], s = cs[h + j];
    const float a = x1 * c, b = x2 * s, e = x2 * c, f = x1 * s;
    x[j] = a - b;
    x[j + h] = e + f;
  }
}

static int kv_quantize_write_impl(int T, int Hq, int Hkv, int D, int bs, int nb,
                                  const uint16_t* key, const uint16_t* value,
                                  const uint16_t* query, int8_t* q_int8, float* q_scale,
                                  const int32_t* slot_mapping, const int32_t* positions,
                                  const float* cos_sin, int R, int max_position,
                                  int8_t* k_cache, int8_t* v_cache, float* k_scale,
                                  float* v_scale) {
  if (T < 0 || !geometry_ok(Hq, Hkv, D, bs, nb)) return -1;
  if (query && (!q_int8 || !q_scale)) return -1;
  if (positions && (!cos_sin || R < 2 || R > D || R % 2 || max_position <= 0)) return -1;
  for (int t = 0; positions && t < T; ++t)
    if (positions[t] < 0 || positions[t] >= max_position) return -3;
  Cache c{Hq, Hkv, D, bs, nb, k_cache, v_cache, k_scale, v_scale};
  std::vector<float> x(D);
  std::vector<int8_t> q(D);
  for (int t = 0; t < T; ++t) {
    const float* cs = positions ? cos_sin + (size_t)positions[t] * R : nullptr;
    /* Query: rotated, then quantized once per (token, q head) and kept for
     * reuse [KV 2.2]. */
    if (query) {
      for (int h = 0; h < Hq; ++h) {
        const uint16_t* src = query + ((size_t)t * Hq + h) * D;
        for (int d = 0; d < D; ++d) x[d] = bf16_to_float(src[d]);
        if (cs) rope_rotate(x.data(), R, cs);
        orc_quantize(x.data(), D, q_int8 + ((size_t)t * Hq + h) * D,
                     q_scale + (size_t)t * Hq + h);
      }
    }
    const int32_t slot = slot_mapping[t];
    if (slot < 0) continue;
    if ((int64_t)slot >= (int64_t)nb * bs) return -2;
    const int blk = slot / bs, off = slot % bs;
    for (int h = 0; h < Hkv; ++h) {
      float s = 0.0f;
      const uint16_t* ks = key + ((size_t)t * Hkv + h) * D;
      for (int d = 0; d < D; ++d) x[d] = bf16_to_float(ks[d]);
      if (cs) rope_rotate(x.data(), R, cs);
      orc_quantize(x.data(), D, q.data(), &s);
      for (int d = 0; d < D; ++d) k_cache[c.k_index(blk, h, off, d)] = q[d];
      k_scale[c.s_index(blk, h, off)] = s;

      const uint16_t* vs = value + ((size_t)t * Hkv + h) * D;
      for (int d = 0; d < D; ++d) x[d] = bf16_to_float(vs[d]);
      orc_quantize(x.data(), D, q.data(), &s);
      for (int d = 0; d < D; ++d) v_cache[c.v_index(blk, h, off, d)] = q[d];
      v_scale[c.s_index(blk, h, off)] = s;
    }
  }
  return 0;
}

/* The bf16 rounding of the BF16-PV ablation, alone (for the pins). */
void orc_round_bf16(const float* x, int n, float* y) {
  for (int i = 0; i < n; ++i) y[i] = round_to_bf16(x[i]);
}

int orc_kv_quantize_write(int T, int Hq, int Hkv, int D, int bs, int nb,
                          const uint16_t* key, const uint16_t* value,
                          const uint16_t* query, int8_t* q_int8, float* q_scale,
                          const int32_t* slot_mapping, int8_t* k_cache,
                          int8_t* v_cache, float* k_scale, float* v_scale) {
  return kv_quantize_write_impl(T, Hq, Hkv, D, bs, nb, key, value, query, q_int8, q_scale,
                                slot_mapping, nullptr, nullptr, 0, 0, k_cache, v_cache, k_scale,
                                v_scale);
}

int orc_kv_quantize_write_rope(int T, int Hq, int Hkv, int D, int bs, int nb,
                               const uint16_t* key, const uint16_t* value,
                               const uint16_t* query, int8_t* q_int8, float* q_scale,
                               const int32_t* slot_mapping, const int32_t* positions,
                               const float* cos_sin, int rotary_dim, int max_position,
                               int8_t* k_cache, int8_t* v_cache, float* k_scale,
                               float* v_scale) {
  if (!positions) return -1;
  return kv_quantize_write_impl(T, Hq, Hkv, D, bs, nb, key, value, query, q_int8, q_scale,
                                slot_mapping, positions, cos_sin, rotary_dim, max_position,
                                k_cache, v_cache, k_scale, v_scale);
}

/* The rotation alone (for the pins): x [n, D] fp32 in place, pos [n]. */
int orc_rope_rotate(int n, int D, float* x, const int32_t* positions, const float* cos_sin,
                    int rotary_dim, int max_position) {
  if (n < 0 || rotary_dim < 2 || rotary_dim > D || rotary_dim % 2) return -1;
  for (int i = 0; i < n; ++i) {
    if (positions[i] < 0 || positions[i] >= max_position) return -3;
    rope_rotate(x + (size_t)i * D, rotary_dim, cos_sin + (size_t)positions[i] * rotary_dim);
  }
  return 0;
}

namespace {

int decode_head_impl(int Hq, int Hkv, int D, int bs, int nb, int seq, int head,
                     const int8_t* q_int8, const float* q_scale, const uint16_t* q_bf16,
                     const int8_t* k_cache, const int8_t* v_cache,
                     const float* k_scale, const float* v_scale,
                     const int32_t* block_tables, int max_blocks,
                     const int32_t* seq_lens, int partition, int w_group,
                     float softmax_scale, int flags, const orc_decode_trace* tr,
                     float* out) {
  if (!geometry_ok(Hq, Hkv, D, bs, nb) || w_group <= 0 || partition <= 0 ||
      partition % w_group != 0)
    return -1;
  const int L = seq_lens[seq];
  if (L < 0 || (L + bs - 1) / bs > max_blocks) return -2;
  if (L == 0) {
    for (int d = 0; d < D; ++d) out[d] = 0.0f;
    return 0;
  }
  Cache c{Hq, Hkv, D, bs, nb, k_cache, v_cache, k_scale, v_scale};
  SeqView sv{&c, block_tables + (size_t)seq * max_blocks, head / (Hq / Hkv)};
  const size_t qr = (size_t)seq * Hq + head;
  const Query q = q_bf16 ? Query{nullptr, 0.0f, q_bf16 + qr * D}
                         : Query{q_int8 + qr * D, q_scale[qr], nullptr};
  const bool exact = (flags & ORC_EXACT) != 0;
  const bool bf16_pv = (flags & ORC_BF16_PV) != 0;
  const bool u8_w = (flags & ORC_UINT8_W) != 0;
  const bool quant_w = (flags & ORC_NO_WQUANT) == 0 && !bf16_pv;

  std::vector<int32_t> acc(L);
  std::vector<float> s(L);
  std::vector<double> s64(L);
  for (int i = 0; i < L; ++i) {
    q.score(sv, i, D, softmax_scale, &s[i], &s64[i], &acc[i]);
    if (tr && tr->acc) tr->acc[i] = acc[i];
    if (tr && tr->s) tr->s[i] = s[i];
  }

  /* [PV 2.2] 256-token partitions, each with its own max m_g and sum l_g,
   * probabilities normalized inside the partition; W = P * sV. */
  const int NP = (L + partition - 1) / partition;
  std::vector<double> m_part(NP), l_part(NP);
  std::vector<double> o_part((size_t)NP * D, 0.0);
  for (int p = 0; p < NP; ++p) {
    const int i0 = p * partition, i1 = std::min(L, i0 + partition), n = i1 - i0;
    double* o = &o_part[(size_t)p * D];
    if (exact) {
      double m = -std::numeric_limits<double>::infinity();
      for (int i = i0; i < i1; ++i) m = std::max(m, s64[i]);
      double l = 0.0;
      std::vector<double> e(n);
      for (int i = 0; i < n; ++i) l += (e[i] = std::exp(s64[i0 + i] - m));
      std::vector<double> W(n);
      for (int i = 0; i < n; ++i) W[i] = e[i] / l * (double)sv.sv(i0 + i);
      for (int g0 = 0; g0 < n; g0 += w_group)
        add_group_plain(&W[g0], i0 + g0, std::min(w_group, n - g0), sv, D, 1.0, o);
      m_part[p] = m;
      l_part[p] = l;
      continue;
    }
    float m = -std::numeric_limits<float>::infinity();
    for (int i = i0; i < i1; ++i) m = std::max(m, s[i]);
    std::vector<float> e(n), P(n), W(n);
    double lsum = 0.0;
    for (int i = 0; i < n; ++i) {
      e[i] = orc_expf(s[i0 + i] - m);
      lsum += (double)e[i];
    }
    const float l = (float)lsum;
    for (int i = 0; i < n; ++i) {
      P[i] = e[i] / l;
      W[i] = P[i] * sv.sv(i0 + i);
      /* BF16-PV ablation: the same W, rounded to bf16, times the int8 V. */
      if (bf16_pv) W[i] = round_to_bf16(W[i]);
    }
    if (tr && tr->P) std::memcpy(tr->P + i0, P.data(), n * sizeof(float));
    if (tr && tr->W) std::memcpy(tr->W + i0, W.data(), n * sizeof(float));
    /* [PV 1, 4] groups of G consecutive tokens, aligned to absolute position. */
    for (int g0 = 0; g0 < n; g0 += w_group) {
      const int gn = std::min(w_group, n - g0);
      if (quant_w && u8_w) {
        add_group_quantized_u8(&W[g0], i0 + g0, gn, sv, D, 1.0, o,
                               tr && tr->Wq ? tr->Wq + i0 + g0 : nullptr,
                               tr && tr->sW ? tr->sW + (i0 + g0) / w_group : nullptr);
      } else if (quant_w) {
        add_group_quantized(&W[g0], i0 + g0, gn, sv, D, 1.0, o,
                            tr && tr->Wq ? tr->Wq + i0 + g0 : nullptr,
                            tr && tr->sW ? tr->sW + (i0 + g0) / w_group : nullptr);
      } else {
        add_group_plain(&W[g0], i0 + g0, gn, sv, D, 1.0, o);
      }
    }
    m_part[p] = m;
    l_part[p] = l;
    if (tr && tr->m) tr->m[p] = m;
    if (tr && tr->l) tr->l[p] = l;
  }
  if (tr && tr->o) std::memcpy(tr->o, o_part.data(), o_part.size() * sizeof(double));

  /* [PV 2.2] merge the partitions with log-sum-exp weights:
   * M = max m_p, w_p = l_p * exp(m_p - M), O = sum w_p o_p / sum w_p. */
  double M = -std::numeric_limits<double>::infinity();
  for (int p = 0; p < NP; ++p) M = std::max(M, m_part[p]);
  std::vector<double> O(D, 0.0);
  double wsum = 0.0;
  for (int p = 0; p < NP; ++p) {
    const double w = l_part[p] * std::exp(m_part[p] - M);
    wsum += w;
    for (int d = 0; d < D; ++d) O[d] += w * o_part[(size_t)p * D + d];
  }
  for (int d = 0; d < D; ++d) out[d] = (float)(O[d] / wsum);
  return 0;
}

int paged_decode_impl(int Hq, int Hkv, int D, int bs, int nb, int S, const int8_t* q_int8,
                      const float* q_scale, const uint16_t* q_bf16, const int8_t* k_cache,
                      const int8_t* v_cache, const float* k_scale, const float* v_scale,
                      const int32_t* block_tables, int max_blocks, const int32_t* seq_lens,
                      int partition, int w_group, float softmax_scale, int flags, float* out) {
  for (int b = 0; b < S; ++b)
    for (int h = 0; h < Hq; ++h) {
      int rc = decode_head_impl(Hq, Hkv, D, bs, nb, b, h, q_int8, q_scale, q_bf16, k_cache,
                                v_cache, k_scale, v_scale, block_tables, max_blocks, seq_lens,
                                partition, w_group, softmax_scale, flags, nullptr,
                                out + ((size_t)b * Hq + h) * D);
      if (rc) return rc;
    }
  return 0;
}

}  // namespace

int orc_decode_head(int Hq, int Hkv, int D, int bs, int nb, int seq, int head,
                    const int8_t* q_int8, const float* q_scale,
                    const int8_t* k_cache, const int8_t* v_cache,
                    const float* k_scale, const float* v_scale,
                    const int32_t* block_tables, int max_blocks,
                    const int32_t* seq_lens, int partition, int w_group,
                    float softmax_scale, int flags, const orc_decode_trace* tr,
                    float* out) {
  return decode_head_impl(Hq, Hkv, D, bs, nb, seq, head, q_int8, q_scale, nullptr, k_cache,
                          v_cache, k_scale, v_scale, block_tables, max_blocks, seq_lens,
                          partition, w_group, softmax_scale, flags, tr, out);
}

int orc_paged_decode(int Hq, int Hkv, int D, int bs, int nb, int S,
                     const int8_t* q_int8, const float* q_scale,
                     const int8_t* k_cache, const int8_t* v_cache,
                     const float* k_scale, const float* v_scale,
                     const int32_t* block_tables, int max_blocks,
                     const int32_t* seq_lens, int partition, int w_group,
                     float softmax_scale, int flags, float* out) {
  return paged_decode_impl(Hq, Hkv, D, bs, nb, S, q_int8, q_scale, nullptr, k_cache, v_cache,
                           k_scale, v_scale, block_tables, max_blocks, seq_lens, partition,
                           w_group, softmax_scale, flags, out);
}

int orc_paged_decode_bf16qk(int Hq, int Hkv, int D, int bs, int nb, int S,
                            const uint16_t* q_bf16, const int8_t* k_cache,
                            const int8_t* v_cache, const float* k_scale, const float* v_scale,
                            const int32_t* block_tables, int max_blocks,
                            const int32_t* seq_lens, int partition, int w_group,
                            float softmax_scale, int flags, float* out) {
  if (!q_bf16) return -1;
  return paged_decode_impl(Hq, Hkv, D, bs, nb, S, nullptr, nullptr, q_bf16, k_cache, v_cache,
                           k_scale, v_scale, block_tables, max_blocks, seq_lens, partition,
                           w_group, softmax_scale, flags, out);
}

namespace {

int prefill_row_impl(int Hq, int Hkv, int D, int bs, int nb, int S, int Tq,
                     int row, int head, const int8_t* q_int8,
                     const float* q_scale, const uint16_t* q_bf16,
                     const int32_t* query_start_loc,
                     const int32_t* seq_lens, const int8_t* k_cache,
                     const int8_t* v_cache, const float* k_scale,
                     const float* v_scale, const int32_t* block_tables,
                     int max_blocks, int tile, int w_group, float softmax_scale,
                     int flags, const orc_prefill_trace* tr, float* out) {
  if (!geometry_ok(Hq, Hkv, D, bs, nb) || w_group <= 0 || tile <= 0 ||
      tile % w_group != 0 || row < 0 || row >= Tq)
    return -1;
  int b = 0;
  while (b < S && query_start_loc[b + 1] <= row) ++b;
  if (b >= S) return -2;
  const int chunk = query_start_loc[b + 1] - query_start_loc[b];
  const int ctx = seq_lens[b] - chunk;
  if (ctx < 0 || (seq_lens[b] + bs - 1) / bs > max_blocks) return -2;
  /* Causal within the chunk: the query at absolute position ctx + j sees keys
   * 0 .. ctx + j, history and chunk alike [KV 3.2]. */
  const int pos = ctx + (row - query_start_loc[b]);
  const int nk = pos + 1;

  Cache c{Hq, Hkv, D, bs, nb, k_cache, v_cache, k_scale, v_scale};
  SeqView sv{&c, block_tables + (size_t)b * max_blocks, head / (Hq / Hkv)};
  const size_t qr = (size_t)row * Hq + head;
  const Query q = q_bf16 ? Query{nullptr, 0.0f, q_bf16 + qr * D}
                         : Query{q_int8 + qr * D, q_scale[qr], nullptr};
  const bool exact = (flags & ORC_EXACT) != 0;
  const bool bf16_pv = (flags & ORC_BF16_PV) != 0;
  const bool u8_w = (flags & ORC_UINT8_W) != 0;
  const bool quant_w = (flags & ORC_NO_WQUANT) == 0 && !bf16_pv;

  /* [PV 2.1] online softmax over key tiles: state (m, l, o). */
  std::vector<double> o(D, 0.0);
  double l = 0.0;
  float m = -std::numeric_limits<float>::infinity();
  double m64 = -std::numeric_limits<double>::infinity();
  for (int t0 = 0, ti = 0; t0 < nk; t0 += tile, ++ti) {
    const int n = std::min(tile, nk - t0);
    std::vector<float> s(n);
    std::vector<double> s64(n);
    for (int j = 0; j < n; ++j) {
      int32_t a;
      q.score(sv, t0 + j, D, softmax_scale, &s[j], &s64[j], &a);
      if (tr && tr->s) tr->s[t0 + j] = s[j];
    }
    if (exact) {
      double mt = m64;
      for (int j = 0; j < n; ++j) mt = std::max(mt, s64[j]);
      const double alpha = std::isinf(m64) ? 0.0 : std::exp(m64 - mt);
      std::vector<double> W(n);
      double psum = 0.0;
      for (int j = 0; j < n; ++j) {
        const double pt = std::exp(s64[j] - mt);
        psum += pt;
        W[j] = pt * (double)sv.sv(t0 + j);
      }
      for (int d = 0; d < D; ++d) o[d] *= alpha;
      for (int g0 = 0; g0 < n; g0 += w_group)
        add_group_plain(&W[g0], t0 + g0, std::min(w_group, n - g0), sv, D, 1.0, o.data());
      l = alpha * l + psum;
      m64 = mt;
      continue;
    }
    /* m' = max(m, max s); alpha = exp(m - m'); p~ = exp(s - m'). */
    float mt = m;
    for (int j = 0; j < n; ++j) mt = std::max(mt, s[j]);
    const float alpha = std::isinf(m) ? 0.0f : orc_expf(m - mt);
    std::vector<float> pt(n), W(n);
    double psum = 0.0;
    for (int j = 0; j < n; ++j) {
      pt[j] = orc_expf(s[j] - mt);
      psum += (double)pt[j];
      /* [PV 2.1] prefill quantizes the unnormalized W = p~ * sV. */
      W[j] = pt[j] * sv.sv(t0 + j);
      /* BF16-PV ablation: the same W rounded to bf16, times the int8 V. */
      if (bf16_pv) W[j] = round_to_bf16(W[j]);
    }
    if (tr && tr->ptil) std::memcpy(tr->ptil + t0, pt.data(), n * sizeof(float));
    /* o = alpha * o + sum p~ sV Vq ; l = alpha * l + sum p~ (unquantized p~). */
    for (int d = 0; d < D; ++d) o[d] *= (double)alpha;
    for (int g0 = 0; g0 < n; g0 += w_group) {
      const int gn = std::min(w_group, n - g0);
      if (quant_w && u8_w) {
        /* [PV 6] the UINT8 candidate: W >= 0, so 0..255 against max W / 255 */
        add_group_quantized_u8(&W[g0], t0 + g0, gn, sv, D, 1.0, o.data(),
                               tr && tr->Wq ? tr->Wq + t0 + g0 : nullptr,
                               tr && tr->sW ? tr->sW + (t0 + g0) / w_group : nullptr);
      } else if (quant_w) {
        add_group_quantized(&W[g0], t0 + g0, gn, sv, D, 1.0, o.data(),
                            tr && tr->Wq ? tr->Wq + t0 + g0 : nullptr,
                            tr && tr->sW ? tr->sW + (t0 + g0) / w_group : nullptr);
      } else {
        add_group_plain(&W[g0], t0 + g0, gn, sv, D, 1.0, o.data());
      }
    }
    l = (double)alpha * l + psum;
    m = mt;
    if (tr && tr->m_tile) tr->m_tile[ti] = m;
  }
  if (tr && tr->l) tr->l[0] = l;
  /* O = o / l after the last tile. */
  for (int d = 0; d < D; ++d) out[d] = (float)(o[d] / l);
  return 0;
}

int prefix_prefill_impl(int Hq, int Hkv, int D, int bs, int nb, int S, int Tq,
                        const int8_t* q_int8, const float* q_scale, const uint16_t* q_bf16,
                        const int32_t* query_start_loc, const int32_t* seq_lens,
                        const int8_t* k_cache, const int8_t* v_cache, const float* k_scale,
                        const float* v_scale, const int32_t* block_tables, int max_blocks,
                        int tile, int w_group, float softmax_scale, int flags,
                        const int32_t* rows, int nrows, float* out) {
  const int n = rows ? nrows : Tq;
  for (int r = 0; r < n; ++r) {
    const int row = rows ? rows[r] : r;
    for (int h = 0; h < Hq; ++h) {
      int rc = prefill_row_impl(Hq, Hkv, D, bs, nb, S, Tq, row, h, q_int8, q_scale, q_bf16,
                                query_start_loc, seq_lens, k_cache, v_cache, k_scale, v_scale,
                                block_tables, max_blocks, tile, w_group, softmax_scale, flags,
                                nullptr, out + ((size_t)row * Hq + h) * D);
      if (rc) return rc;
    }
  }
  return 0;
}

}  // namespace

int orc_prefill_row(int Hq, int Hkv, int D, int bs, int nb, int S, int Tq,
                    int row, int head, const int8_t* q_int8,
                    const float* q_scale, const int32_t* query_start_loc,
                    const int32_t* seq_lens, const int8_t* k_cache,
                    const int8_t* v_cache, const float* k_scale,
                    const float* v_scale, const int32_t* block_tables,
                    int max_blocks, int tile, int w_group, float softmax_scale,
                    int flags, const orc_prefill_trace* tr, float* out) {
  return prefill_row_impl(Hq, Hkv, D, bs, nb, S, Tq, row, head, q_int8, q_scale, nullptr,
                          query_start_loc, seq_lens, k_cache, v_cache, k_scale, v_scale,
                          block_tables, max_blocks, tile, w_group, softmax_scale, flags, tr,
                          out);
}

int orc_prefix_prefill(int Hq, int Hkv, int D, int bs, int nb, int S, int Tq,
                       const int8_t* q_int8, const float* q_scale,
                       const int32_t* query_start_loc, const int32_t* seq_lens,
                       const int8_t* k_cache, const int8_t* v_cache,
                       const float* k_scale, const float* v_scale,
                       const int32_t* block_tables, int max_blocks, int tile,
                       int w_group, float softmax_scale, int flags,
                       const int32_t* rows, int nrows, float* out) {
  return prefix_prefill_impl(Hq, Hkv, D, bs, nb, S, Tq, q_int8, q_scale, nullptr,
                             query_start_loc, seq_lens, k_cache, v_cache, k_scale, v_scale,
                             block_tables, max_blocks, tile, w_group, softmax_scale, flags, rows,
                             nrows, out);
}

int orc_prefix_prefill_bf16qk(int Hq, int Hkv, int D, int bs, int nb, int S, int Tq,
                              const uint16_t* q_bf16, const int32_t* query_start_loc,
                              const int32_t* seq_lens, const int8_t* k_cache,
                              const int8_t* v_cache, const float* k_scale,
                              const float* v_scale, const int32_t* block_tables,
                              int max_blocks, int tile, int w_group, float softmax_scale,
                              int flags, const int32_t* rows, int nrows, float* out) {
  if (!q_bf16) return -1;
  return prefix_prefill_impl(Hq, Hkv, D, bs, nb, S, Tq, nullptr, nullptr, q_bf16,
                             query_start_loc, seq_lens, k_cache, v_cache, k_scale, v_scale,
                             block_tables, max_blocks, tile, w_group, softmax_scale, flags, rows,
                             nrows, out);
}

}  // extern "C"
