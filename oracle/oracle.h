/*
 * CPU oracle for paged attention over an INT8 KV cache.
 *
 * TEST INFRASTRUCTURE ONLY.  This is the slow, plain, single-threaded
 * definition of what the GPU path must compute.  Only the test suite, the
 * package's smoke check and the benchmark's CPU-baseline leg may load it; the
 * product path never does.  It shares no code, header or table with the HIP
 * library.
 *
 * Sources (pages, by title):
 *  [KV]  "INT8 KV and INT8 MMAC attention inference optimisation on a gfx936
 *        DCU" (part 1 of the series): per-token/per-head symmetric quantization
 *        (section 2.1), fused producer and paged write (2.2), cache layouts
 *        (2.3), decode consumption (3.3), prefill-with-history (3.2).
 *  [PV]  "Implementing INT8 PV MMAC on a gfx936 DCU: V-scale fusion,
 *        probability quantization, fragment grouping" (part 3): V-scale folding
 *        and W-group quantization (section 1), online-softmax forms for
 *        prefill (2.1) and decode (2.2), operand roles and the int32 bound (3),
 *        group/fragment agreement (4).
 *
 * Precision: elementwise quantities (scores, exponentials, probabilities, W,
 * scales) are fp32, as the pages' sketches are; the exponential of an fp32
 * argument is the correctly rounded fp32 value of e^x.  Reductions (l, o and
 * the partition merge) accumulate in fp64 so that the result does not depend
 * on summation order.  Integer dot products are exact.
 *
 * Status: every function returns 0 on success and a negative value on a
 * rejected argument; nothing is allocated that outlives a call.
 */
#ifndef I8KV_ORACLE_H
#define I8KV_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Flags for the attention functions. */
enum {
  ORC_NO_WQUANT = 1, /* PV uses W itself (no group quantization) */
  ORC_EXACT = 2,     /* scores, exp, P and W in fp64 and W unquantized: exact
                        softmax attention over the dequantized int8 cache */
  ORC_BF16_PV = 4,   /* the BF16-PV ablation -- W (decode: P * sV; prefill:
                        p~ * sV) rounded to bf16 (nearest, ties to even)
                        instead of group-quantized to int8, times the int8 V
                        (exact products, fp64 sum); everything else unchanged */
  ORC_UINT8_W = 8    /* W groups quantized to UINT8 (sW = max W / 255, Wq in
                        [0, 255]), decode and prefill; the trace's Wq holds
                        the uint8 codes */
};

/* Symmetric int8 quantization of one vector [KV 2.1]:
 * amax = max|x|, scale = amax/127, q = clamp(round(x/scale), -127, 127),
 * rounding half away from zero; amax == 0 gives scale 0 and q = 0. */
void orc_quantize(const float* x, int n, int8_t* q, float* scale);

/* Quantization of one W group [PV 1]: sW = max W / 127, Wq = round(W/sW). */
void orc_quantize_w(const float* w, int n, int8_t* wq, float* sw);

/* The UINT8 variant: sW = max W / 255, Wq = round(W/sW) in [0, 255]. */
void orc_quantize_w_u8(const float* w, int n, uint8_t* wq, float* sw);

/* fp32 -> nearest bf16 (ties to even), returned as fp32; finite inputs. */
void orc_round_bf16(const float* x, int n, float* y);

/* Producer [KV 2.2, 2.3]: quantize K and V per (token, KV head) and write
 * them to the pages at slot_mapping[t] (< 0: skip); quantize Q per
 * (token, q head) when query != NULL.
 *   key, value  [T, Hkv, D] bf16 bits;  query [T, Hq, D] bf16 bits or NULL
 *   q_int8 [T, Hq, D], q_scale [T, Hq]
 *   k_cache [nb, Hkv, D/16, bs, 16], v_cache [nb, Hkv, D, bs] int8
 *   k_scale, v_scale [nb, bs, Hkv] fp32 */
int orc_kv_quantize_write(int T, int Hq, int Hkv, int D, int bs, int nb,
                          const uint16_t* key, const uint16_t* value,
                          const uint16_t* query, int8_t* q_int8, float* q_scale,
                          const int32_t* slot_mapping, int8_t* k_cache,
                          int8_t* v_cache, float* k_scale, float* v_scale);

/* Producer with rotary position embedding of Q and K before quantization
 * ([KV 2.2] step 2).  The pages name the step but not its variant; the
 * reading taken is the rotate-half pairing over the first R = rotary_dim
 * dims: for j < R/2 the pair (x[j], x[j + R/2]) turns by the angle whose
 * cosine and sine the caller tabulates per position,
 *   c = cos_sin[pos][j], s = cos_sin[pos][R/2 + j],
 *   x'[j] = x[j] c - x[j + R/2] s,  x'[j + R/2] = x[j + R/2] c + x[j] s,
 * each product and the difference / sum rounded to fp32 on its own (no fused
 * multiply-add); dims R..D-1 pass unchanged.  V is not rotated.
 *   positions [T] int32 in [0, max_position) (else -3)
 *   cos_sin [max_position, R] fp32 */
int orc_kv_quantize_write_rope(int T, int Hq, int Hkv, int D, int bs, int nb,
                               const uint16_t* key, const uint16_t* value,
                               const uint16_t* query, int8_t* q_int8, float* q_scale,
                               const int32_t* slot_mapping, const int32_t* positions,
                               const float* cos_sin, int rotary_dim, int max_position,
                               int8_t* k_cache, int8_t* v_cache, float* k_scale,
                               float* v_scale);

/* The rotation of orc_kv_quantize_write_rope alone, in place on n fp32
 * vectors of D values (x [n, D]) at positions [n]. */
int orc_rope_rotate(int n, int D, float* x, const int32_t* positions, const float* cos_sin,
                    int rotary_dim, int max_position);

/* Per-(seq, q head) record of the decode computation. All pointers may be
 * NULL. L = seq_len, NP = ceil(L/partition), NG = number of W groups. */
typedef struct {
  float* s;       /* [L]  fp32 scores */
  float* P;       /* [L]  partition-normalized probabilities */
  float* W;       /* [L]  P * sV */
  int8_t* Wq;     /* [L]  quantized W */
  float* sW;      /* [NG] group scales, groups in token order */
  float* m;       /* [NP] partition max */
  float* l;       /* [NP] partition exp-sum (fp32) */
  double* o;      /* [NP*D] partition outputs */
  int32_t* acc;   /* [L]  int32 QK accumulators */
} orc_decode_trace;

/* Paged decode [KV 3.3; PV 2.2]: one query per sequence.
 *   q_int8 [S, Hq, D], q_scale [S, Hq], block_tables [S, max_blocks],
 *   seq_lens [S]; out [S, Hq, D] fp32. */
int orc_paged_decode(int Hq, int Hkv, int D, int bs, int nb, int S,
                     const int8_t* q_int8, const float* q_scale,
                     const int8_t* k_cache, const int8_t* v_cache,
                     const float* k_scale, const float* v_scale,
                     const int32_t* block_tables, int max_blocks,
                     const int32_t* seq_lens, int partition, int w_group,
                     float softmax_scale, int flags, float* out);

/* BF16-QK ablation of orc_paged_decode: the query is q_bf16 [S, Hq, D] (bf16
 * bits, not quantized) against the int8 K codes; score = ((float)dot * sK) *
 * softmax_scale with dot = sum_d q[d] * k8[d] summed in fp64 and rounded once
 * to fp32 (fp64 throughout under ORC_EXACT).  Everything after the scores is
 * orc_paged_decode's, flags included. */
int orc_paged_decode_bf16qk(int Hq, int Hkv, int D, int bs, int nb, int S,
                            const uint16_t* q_bf16, const int8_t* k_cache,
                            const int8_t* v_cache, const float* k_scale, const float* v_scale,
                            const int32_t* block_tables, int max_blocks,
                            const int32_t* seq_lens, int partition, int w_group,
                            float softmax_scale, int flags, float* out);

/* Same computation for one (seq, q head), filling `trace`; out [D]. */
int orc_decode_head(int Hq, int Hkv, int D, int bs, int nb, int seq, int head,
                    const int8_t* q_int8, const float* q_scale,
                    const int8_t* k_cache, const int8_t* v_cache,
                    const float* k_scale, const float* v_scale,
                    const int32_t* block_tables, int max_blocks,
                    const int32_t* seq_lens, int partition, int w_group,
                    float softmax_scale, int flags, const orc_decode_trace* trace,
                    float* out);

/* Per-(row, q head) record of the prefill computation. */
typedef struct {
  float* s;       /* [nk] scores of visible keys (nk = position + 1) */
  float* ptil;    /* [nk] p~ as used (relative to the running max) */
  int8_t* Wq;     /* [nk] */
  float* sW;      /* [ceil(nk/G)] */
  float* m_tile;  /* [ceil(nk/tile)] running max after each tile */
  double* l;      /* [1] final l */
} orc_prefill_trace;

/* Chunked prefill with history [KV 3.2; PV 2.1]: one online softmax over the
 * history plus the causal chunk.  Query row j of sequence b (rows
 * query_start_loc[b] .. query_start_loc[b+1]-1) sits at absolute position
 * seq_lens[b] - chunk_b + (j - query_start_loc[b]) and sees keys 0..position.
 *   q_int8 [Tq, Hq, D], q_scale [Tq, Hq]; out [Tq, Hq, D].
 * rows/nrows: if rows != NULL only those query rows are computed (others of
 * `out` are left untouched). */
int orc_prefix_prefill(int Hq, int Hkv, int D, int bs, int nb, int S, int Tq,
                       const int8_t* q_int8, const float* q_scale,
                       const int32_t* query_start_loc, const int32_t* seq_lens,
                       const int8_t* k_cache, const int8_t* v_cache,
                       const float* k_scale, const float* v_scale,
                       const int32_t* block_tables, int max_blocks, int tile,
                       int w_group, float softmax_scale, int flags,
                       const int32_t* rows, int nrows, float* out);

int orc_prefill_row(int Hq, int Hkv, int D, int bs, int nb, int S, int Tq,
                    int row, int head, const int8_t* q_int8,
                    const float* q_scale, const int32_t* query_start_loc,
                    const int32_t* seq_lens, const int8_t* k_cache,
                    const int8_t* v_cache, const float* k_scale,
                    const float* v_scale, const int32_t* block_tables,
                    int max_blocks, int tile, int w_group, float softmax_scale,
                    int flags, const orc_prefill_trace* trace, float* out);

/* BF16-QK ablation of orc_prefix_prefill: q_bf16 [Tq, Hq, D] bf16 bits, scores
 * as in orc_paged_decode_bf16qk, the rest unchanged. */
int orc_prefix_prefill_bf16qk(int Hq, int Hkv, int D, int bs, int nb, int S, int Tq,
                              const uint16_t* q_bf16, const int32_t* query_start_loc,
                              const int32_t* seq_lens, const int8_t* k_cache,
                              const int8_t* v_cache, const float* k_scale,
                              const float* v_scale, const int32_t* block_tables,
                              int max_blocks, int tile, int w_group, float softmax_scale,
                              int flags, const int32_t* rows, int nrows, float* out);

/* Correctly rounded fp32 exponential used by the oracle. */
float orc_expf(float x);

#ifdef __cplusplus
}
#endif
#endif
