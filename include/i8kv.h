/*
 * i8kv -- paged attention over an INT8 KV cache, native to AMD MI355X (gfx950).
 *
 * C ABI of the library libi8kv.so.  Sixteen calls, on the operations defined on the pages
 *   [KV] "INT8 KV and INT8 MMAC attention inference optimisation on a gfx936
 *        DCU" (part 1 of the series), and
 *   [PV] "Implementing INT8 PV MMAC on a gfx936 DCU: V-scale fusion,
 *        probability quantization, fragment grouping" (part 3):
 *
 *   i8kv_kv_quantize_write  -- the fused KV producer ([KV] sections 2.1-2.3)
 *   i8kv_kv_quantize_write_rope -- the same producer with the rotary
 *                              embedding of Q and K fused in ([KV] 2.2)
 *   i8kv_paged_decode_int8  -- decode over 256-token partitions ([KV] 3.3,
 *                              [PV] 2.2, merge by log-sum-exp weights)
 *   i8kv_paged_decode_partials, i8kv_paged_decode_merge -- the decode's two
 *                              stages as separate calls (partitions, then the
 *                              merge of their partials; [PV] 2.2)
 *   i8kv_paged_decode_int8_noalloc -- the decode for callers that cannot
 *                              allocate (partials in a fixed per-GPU array)
 *   i8kv_prefix_prefill_int8 -- chunked prefill with history in one online
 *                              softmax ([KV] 3.2, [PV] 2.1)
 *   i8kv_decode_step_int8   -- the producer of each sequence's newest token
 *                              fused into the decode of that token
 *   i8kv_paged_decode_bf16pv -- the decode with a bf16 PV product instead of
 *                              the int8 one (the pages' PV ablation, [PV] 5)
 *   i8kv_paged_decode_uint8w -- the decode with UINT8 W groups (the candidate
 *                              of [PV] 6: W >= 0 gets one more bit)
 *   i8kv_paged_decode_ex    -- the decode with options: PV variant, several
 *                              causal queries per sequence, bf16 output
 *   i8kv_prefix_prefill_bf16pv -- the prefill with a bf16 PV product ([PV] 5)
 *   i8kv_paged_decode_bf16qk -- the decode with a bf16 QK product (the
 *                              pages' QK comparison, [KV] 4.1)
 *   i8kv_prefix_prefill_bf16qk -- the prefill with a bf16 QK product ([KV] 4.1)
 *   i8kv_prefix_prefill_uint8w -- the prefill with UINT8 W groups ([PV] 6)
 *   i8kv_prefix_prefill_ex  -- the prefill with options: PV variant, bf16 output
 * plus the workspace-size queries, i8kv_status_string and i8kv_abi_version.
 *
 * Conventions for every call
 *  - Tensor arguments are DEVICE pointers owned by the caller, C-contiguous in
 *    the layouts given below.  The library never allocates, frees or
 *    synchronizes, keeps no global state and is re-entrant; all work is
 *    enqueued on `stream` (NULL = the default stream) and is asynchronous.
 *    The one exception is i8kv_paged_decode_int8_noalloc, whose fixed device
 *    array per GPU is shared by every call on that GPU (see there).
 *  - bf16 tensors are passed as their 16-bit patterns (uint16_t).
 *  - Cache layouts ([KV] 2.3), with x = 16 head-dim bytes per token:
 *      k_cache [num_blocks, Hkv, D/16, block_size, 16]  int8
 *      v_cache [num_blocks, Hkv, D, block_size]         int8
 *      k_scale, v_scale [num_blocks, block_size, Hkv]   fp32
 *    Token position i of a sequence lives in page block_tables[s][i / 16] at
 *    offset i % 16.  Q head h reads KV head h / (Hq / Hkv).
 *  - Quantization ([KV] 2.1): amax = max|x|, scale = amax / 127 (fp32, IEEE
 *    division), q = clamp(round(x / scale), -127, 127), rounding half away
 *    from zero; amax = 0 stores scale 0 and all-zero codes.
 *  - Status: argument and shape checks run on the host BEFORE anything is
 *    enqueued; on any non-OK status nothing has been launched, except
 *    I8KV_ERR_LAUNCH, which reports a failed enqueue.  Before enqueuing,
 *    each call clears the calling thread's pending (non-sticky) HIP error, as
 *    hipGetLastError() would, so that error describes its own launches; a
 *    sticky error (an earlier device fault) is still reported.  No C++
 *    exception crosses the ABI.
 *  - Supported shapes: block_size = 16; head_dim in {64, 128, 256};
 *    Hq % Hkv = 0 with Hq / Hkv <= 16; w_group in {32, 64};
 *    partition_size = 256.  Other values return I8KV_ERR_UNSUPPORTED.
 *  - Preconditions not checked on the host (they live in device memory):
 *    block ids < num_blocks, slots < num_blocks * block_size, finite inputs,
 *    seq_lens[s] <= max_seq_len and <= 16 * max_blocks_per_seq.
 */
#ifndef I8KV_H
#define I8KV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define I8KV_ABI_VERSION 1

typedef enum {
  I8KV_OK = 0,
  I8KV_ERR_NULL = 1,          /* a required pointer is NULL */
  I8KV_ERR_INVALID_ARG = 2,   /* negative count, inconsistent sizes */
  I8KV_ERR_UNSUPPORTED = 3,   /* shape outside the supported set above */
  I8KV_ERR_WORKSPACE = 4,     /* workspace missing or too small */
  I8KV_ERR_LAUNCH = 5         /* the HIP runtime refused the launch */
} i8kv_status;

/* Geometry shared by the cache and the attention calls. */
typedef struct {
  int32_t num_q_heads;   /* Hq */
  int32_t num_kv_heads;  /* Hkv */
  int32_t head_dim;      /* D */
  int32_t block_size;    /* tokens per page; must be 16 */
  int32_t num_blocks;    /* pages in the cache */
} i8kv_cache_desc;

/* hipStream_t, passed as an opaque handle. */
typedef void* i8kv_stream_t;

/*
 * Fused KV producer ([KV] 2.2): for each token t < num_tokens, quantize K and
 * V per (token, KV head) and write codes and scales to slot slot_mapping[t]
 * (page slot / 16, offset slot % 16); a negative slot skips the cache write.
 * When `query` is non-NULL, also quantize Q once per (token, q head) into
 * q_int8 / q_scale, for reuse by every partition that reads it.
 *   key, value   [T, Hkv, D] bf16          query  [T, Hq, D] bf16 or NULL
 *   q_int8       [T, Hq, D] int8           q_scale [T, Hq] fp32
 *   slot_mapping [T] int32
 * Errors: NULL for missing key/value/slot_mapping/cache pointers or for
 * q_int8/q_scale missing while query is given; INVALID_ARG for num_tokens < 0.
 * num_tokens = 0 enqueues nothing.
 */
i8kv_status i8kv_kv_quantize_write(const i8kv_cache_desc* desc, int32_t num_tokens,
                                   const uint16_t* key, const uint16_t* value,
                                   const uint16_t* query, int8_t* q_int8,
                                   float* q_scale, const int32_t* slot_mapping,
                                   int8_t* k_cache, int8_t* v_cache,
                                   float* k_scale, float* v_scale,
                                   i8kv_stream_t stream);

/*
 * The fused KV producer with rotary position embedding ([KV] 2.2 lists RoPE
 * as the producer's second step; the pages do not fix its variant).  Same as
 * i8kv_kv_quantize_write, except that Q and K (not V) are first rotated by
 * their token's position, in the rotate-half pairing over the first
 * R = rotary_dim dims: for j < R/2, with c = cos_sin[pos][j] and
 * s = cos_sin[pos][R/2 + j],
 *   x[j]' = x[j] c - x[j + R/2] s,   x[j + R/2]' = x[j + R/2] c + x[j] s,
 * each product and the difference / sum rounded to fp32 (no fused
 * multiply-add); dims R..D-1 pass unchanged; the rotated fp32 vector is then
 * quantized as above.
 *   positions [T] int32, each in [0, max_position)
 *   cos_sin   [max_position, R] fp32 (cosines, then sines), 4-byte aligned
 * A position outside [0, max_position) is clamped into it on the device (no
 * read leaves the table; the result for that token is then meaningless).
 * Errors: as i8kv_kv_quantize_write; NULL for missing positions / cos_sin;
 * INVALID_ARG for max_position <= 0, rotary_dim <= 0 or a misaligned table;
 * UNSUPPORTED unless rotary_dim <= D and rotary_dim % (2 D / 64) == 0
 * (even for D = 64, a multiple of 4 for D = 128 and of 8 for D = 256).
 */
i8kv_status i8kv_kv_quantize_write_rope(const i8kv_cache_desc* desc, int32_t num_tokens,
                                        const uint16_t* key, const uint16_t* value,
                                        const uint16_t* query, int8_t* q_int8, float* q_scale,
                                        const int32_t* slot_mapping, const int32_t* positions,
                                        const float* cos_sin, int32_t rotary_dim,
                                        int32_t max_position, int8_t* k_cache, int8_t* v_cache,
                                        float* k_scale, float* v_scale, i8kv_stream_t stream);

/*
 * Bytes of device workspace that i8kv_paged_decode_int8 needs for num_seqs
 * sequences of at most max_seq_len tokens: the per-partition partials
 * (m_p, l_p and the partition output), i.e. the partition-merge space that
 * [KV] 5.6 requires to be counted in the memory budget next to the int8
 * pages and their scales.  Returns 0 for invalid arguments.
 */
size_t i8kv_paged_decode_workspace_bytes(const i8kv_cache_desc* desc, int32_t num_seqs,
                                         int32_t max_seq_len, int32_t partition_size);

/*
 * Paged decode over the INT8 cache ([KV] 3.3; [PV] 2.2), one query per
 * sequence attending to its seq_lens[s] cached tokens:
 *   score_i = ((acc_i * sQ) * sK_i) * softmax_scale, acc_i the int32 dot
 *             product of the int8 query and key;
 *   per 256-token partition p: m_p = max score, e_i = exp(score_i - m_p),
 *             l_p = sum e_i, P_i = e_i / l_p, W_i = P_i * sV_i;
 *   per aligned group of w_group tokens: sW = max W / 127, Wq = round(W / sW),
 *             o_p += sW * (Wq x Vq) with an int8 x int8 -> int32 product;
 *   merge:    O = sum_p w_p o_p / sum_p w_p, w_p = l_p exp(m_p - max m).
 *   q_int8 [S, Hq, D], q_scale [S, Hq]   (as written by the producer)
 *   block_tables [S, max_blocks_per_seq] int32, seq_lens [S] int32
 *   out [S, Hq, D] fp32, fully overwritten (seq_len 0 gives zeros)
 * workspace: device memory (256-byte aligned) of at least
 *   i8kv_paged_decode_workspace_bytes(desc, S, max_seq_len, partition_size)
 *   bytes; its contents need no initialization.  Calls that run concurrently
 *   must use different workspaces.  The call enqueues two kernels (partitions,
 *   then the merge, skipped when no sequence spans more than one partition).
 * Errors: NULL, INVALID_ARG (S < 0, max_seq_len < 0, max_seq_len larger than
 * 16 * max_blocks_per_seq), UNSUPPORTED (also max_seq_len > 2^20), WORKSPACE.
 */
i8kv_status i8kv_paged_decode_int8(const i8kv_cache_desc* desc, int32_t num_seqs,
                                   const int8_t* q_int8, const float* q_scale,
                                   const int8_t* k_cache, const int8_t* v_cache,
                                   const float* k_scale, const float* v_scale,
                                   const int32_t* block_tables, int32_t max_blocks_per_seq,
                                   const int32_t* seq_lens, int32_t max_seq_len,
                                   int32_t partition_size, int32_t w_group,
                                   float softmax_scale, void* workspace,
                                   size_t workspace_bytes, float* out,
                                   i8kv_stream_t stream);

/*
 * i8kv_paged_decode_int8 for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments without the workspace, the same kernels and
 * the same output bit for bit.  The per-partition partials go to a fixed
 * device array inside the library, one per GPU, of
 * i8kv_paged_decode_noalloc_max_bytes() = 64 MiB, held from the first call on
 * a GPU until the process ends.  A call whose partials need more
 * (i8kv_paged_decode_workspace_bytes(desc, S, max_seq_len, 256) > 64 MiB; at
 * 24 q / 4 KV heads x 256 that is S * max_seq_len above ~690K tokens, e.g.
 * 16 sequences of up to 32768 fit) returns I8KV_ERR_WORKSPACE before touching
 * the device.  The call allocates and frees
 * nothing.  All calls on one GPU share the array: calls that overlap on one
 * GPU (other streams, other threads) race; serialize them.  The array needs no
 * initialization.  `stream` must belong to the current device.  Errors as for
 * i8kv_paged_decode_int8, and LAUNCH if the array's device address cannot be
 * obtained.
 */
size_t i8kv_paged_decode_noalloc_max_bytes(void);
i8kv_status i8kv_paged_decode_int8_noalloc(const i8kv_cache_desc* desc, int32_t num_seqs,
                                           const int8_t* q_int8, const float* q_scale,
                                           const int8_t* k_cache, const int8_t* v_cache,
                                           const float* k_scale, const float* v_scale,
                                           const int32_t* block_tables,
                                           int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                           int32_t max_seq_len, int32_t partition_size,
                                           int32_t w_group, float softmax_scale, float* out,
                                           i8kv_stream_t stream);

/*
 * The two stages of i8kv_paged_decode_int8 as separate calls ([PV] 2.2: each
 * 256-token partition is reduced on its own to (m_p, l_p, o_p), and the
 * partition outputs are merged with log-sum-exp weights).  Run back to back
 * over one workspace they give the output of i8kv_paged_decode_int8 bit for
 * bit.  Apart, they let the partitions of a sequence be computed where its
 * pages live and merged once (a decode sharded over partitions: a shard that
 * starts at a multiple of 256 tokens is a sequence of its own whose block
 * table starts at its first page, since scores, partition softmax and W
 * groups are relative to the partition).
 *
 * i8kv_paged_decode_partials: the arguments of i8kv_paged_decode_int8
 * without `out`.  Writes, for every sequence s, KV head h, partition
 * p < ceil(seq_lens[s] / 256) and q head j of the KV head's group of
 * g = Hq / Hkv (row r = j), into the workspace:
 *   o  float [S][Hkv][P][g][D] at byte 0:  o_p = sum over the partition's
 *      W groups of sW * (Wq x Vq), P_i normalized by the partition's l_p;
 *   ml float [S][Hkv][P][g][2] at byte align256(S * Hkv * P * g * D * 4):
 *      (m_p, l_p), the partition's max score and sum of exp(score - m_p);
 * with P = ceil(max_seq_len / 256) (the size that
 * i8kv_paged_decode_workspace_bytes(desc, S, max_seq_len, 256) covers).
 * Entries of partitions past a sequence are not written.  Errors as for
 * i8kv_paged_decode_int8.
 *
 * i8kv_paged_decode_merge: reads that workspace (filled by the partials call
 * for the same desc, S and max_seq_len, or assembled by the caller in the
 * same layout) and writes out [S, Hq, D] fp32:
 *   O = sum_p w_p o_p / sum_p w_p,  w_p = l_p exp(m_p - max_p m_p),
 * over p < ceil(seq_lens[s] / 256); a one-partition sequence gets o_0 itself
 * and an empty one zeros.  Errors: NULL (desc, seq_lens, workspace, out),
 * INVALID_ARG / UNSUPPORTED as for i8kv_paged_decode_int8, WORKSPACE.
 */
i8kv_status i8kv_paged_decode_partials(const i8kv_cache_desc* desc, int32_t num_seqs,
                                       const int8_t* q_int8, const float* q_scale,
                                       const int8_t* k_cache, const int8_t* v_cache,
                                       const float* k_scale, const float* v_scale,
                                       const int32_t* block_tables, int32_t max_blocks_per_seq,
                                       const int32_t* seq_lens, int32_t max_seq_len,
                                       int32_t partition_size, int32_t w_group,
                                       float softmax_scale, void* workspace,
                                       size_t workspace_bytes, i8kv_stream_t stream);
i8kv_status i8kv_paged_decode_merge(const i8kv_cache_desc* desc, int32_t num_seqs,
                                    const int32_t* seq_lens, int32_t max_seq_len,
                                    int32_t partition_size, const void* workspace,
                                    size_t workspace_bytes, float* out, i8kv_stream_t stream);

/*
 * The BF16-PV ablation of i8kv_paged_decode_int8 ([PV] 5 compares its int8 PV
 * with a bf16 PV that changes nothing else): the same scores, partitions,
 * softmax and merge, but each partition's PV is
 *   o_p[d] = sum_i bf16(W_i) * Vq_i[d],   W_i = P_i * sV_i,
 * with W rounded to bf16 (nearest, ties to even) instead of group-quantized
 * to int8, the int8 V taken exactly as bf16, and fp32 accumulation
 * (v_mfma_f32_16x16x32_bf16).  Arguments, workspace size and errors as
 * i8kv_paged_decode_int8 without w_group.
 */
i8kv_status i8kv_paged_decode_bf16pv(const i8kv_cache_desc* desc, int32_t num_seqs,
                                     const int8_t* q_int8, const float* q_scale,
                                     const int8_t* k_cache, const int8_t* v_cache,
                                     const float* k_scale, const float* v_scale,
                                     const int32_t* block_tables, int32_t max_blocks_per_seq,
                                     const int32_t* seq_lens, int32_t max_seq_len,
                                     int32_t partition_size, float softmax_scale, void* workspace,
                                     size_t workspace_bytes, float* out, i8kv_stream_t stream);

/*
 * The BF16-QK ablation of i8kv_paged_decode_int8 ([KV] 4.1 compares the int8
 * QK matrix block with a bf16 one): the query is not quantized; its bf16
 * values meet the int8 K codes, taken exactly as bf16, in
 * v_mfma_f32_16x16x32_bf16 with fp32 accumulation, and
 *   score_i = (dot_i * sK_i) * softmax_scale,   dot_i = sum_d q[d] * Kq_i[d].
 * Partitions, softmax, the int8 W groups, PV and the merge are those of
 * i8kv_paged_decode_int8.
 *   query_bf16 [S, Hq, D] bf16 bits (16-byte aligned) in place of q_int8 and
 *   q_scale; every other argument, the workspace size and the errors as
 *   i8kv_paged_decode_int8.
 */
i8kv_status i8kv_paged_decode_bf16qk(const i8kv_cache_desc* desc, int32_t num_seqs,
                                     const uint16_t* query_bf16, const int8_t* k_cache,
                                     const int8_t* v_cache, const float* k_scale,
                                     const float* v_scale, const int32_t* block_tables,
                                     int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                     int32_t max_seq_len, int32_t partition_size,
                                     int32_t w_group, float softmax_scale, void* workspace,
                                     size_t workspace_bytes, float* out, i8kv_stream_t stream);

/*
 * The decode with UINT8 W groups ([PV] 6 lists UINT8 probabilities as the
 * candidate with one more bit, since W = P * sV >= 0, but found no correct
 * and fast UINT8 x INT8 path): as i8kv_paged_decode_int8 except that each
 * aligned group of w_group tokens uses
 *   sW = max W / 255,  Wq = round(W / sW) in [0, 255] (ties away from zero),
 *   o_p += sW * sum_i Wq_i * Vq_i.
 * gfx950 has only a signed int8 MFMA: the kernel feeds Wq - 128 (an int8)
 * and adds 128 * sum_i Vq_i back, the column sums coming from the same MFMA
 * with all-ones rows; the integer result is exact.  Arguments, workspace and
 * errors as i8kv_paged_decode_int8.
 */
i8kv_status i8kv_paged_decode_uint8w(const i8kv_cache_desc* desc, int32_t num_seqs,
                                     const int8_t* q_int8, const float* q_scale,
                                     const int8_t* k_cache, const int8_t* v_cache,
                                     const float* k_scale, const float* v_scale,
                                     const int32_t* block_tables, int32_t max_blocks_per_seq,
                                     const int32_t* seq_lens, int32_t max_seq_len,
                                     int32_t partition_size, int32_t w_group,
                                     float softmax_scale, void* workspace,
                                     size_t workspace_bytes, float* out, i8kv_stream_t stream);

/* PV variants of i8kv_paged_decode_ex. */
enum { I8KV_PV_INT8 = 0, I8KV_PV_BF16 = 1, I8KV_PV_UINT8 = 2 };

typedef struct {
  int32_t partition_size;  /* 256 */
  int32_t w_group;         /* 32 or 64 (unused by I8KV_PV_BF16) */
  float softmax_scale;
  int32_t pv;              /* I8KV_PV_INT8 (the method), _BF16 or _UINT8 (see above) */
  int32_t queries_per_seq; /* nq >= 1, nq * (Hq / Hkv) <= 16 */
  int32_t out_bf16;        /* 0: out is fp32; 1: out is bf16 bits (nearest, ties to even) */
} i8kv_decode_opts;

/* Workspace bytes of i8kv_paged_decode_ex: the partition-merge space of its
 * nq * (Hq / Hkv) rows per KV head, for the memory budget of [KV] 5.6
 * (0 for invalid arguments). */
size_t i8kv_paged_decode_ex_workspace_bytes(const i8kv_cache_desc* desc,
                                            const i8kv_decode_opts* opts, int32_t num_seqs,
                                            int32_t max_seq_len);

/*
 * The decode with options, in the serving shapes the pages' decode call is
 * used in ([KV] 3.3 outputs bf16; several new tokens per sequence):
 *  - nq = queries_per_seq queries per sequence, at positions
 *    L - nq .. L - 1 (L = seq_lens[s]); query j attends causally to keys
 *    0 .. L - nq + j, and each is computed exactly as a one-query decode of
 *    the sequence cut after its own position (256-token partitions of that
 *    prefix, the same W groups, the same merge); K and V are read once for
 *    all nq queries.  A query that sees no key (L < nq) outputs zeros.
 *      q_int8 [S * nq, Hq, D], q_scale [S * nq, Hq]   (row s * nq + j)
 *      out    [S * nq, Hq, D]
 *  - pv: the method's int8 W groups, the BF16-PV ablation or UINT8 W.
 *  - out_bf16: the fp32 result rounded to bf16 (nearest, ties to even).
 * Workspace: i8kv_paged_decode_ex_workspace_bytes(desc, opts, S, max_seq_len).
 * Errors: as i8kv_paged_decode_int8; NULL for opts; INVALID_ARG for nq < 1
 * or out_bf16 not 0/1; UNSUPPORTED for nq * Hq/Hkv > 16 or an unknown pv.
 */
i8kv_status i8kv_paged_decode_ex(const i8kv_cache_desc* desc, const i8kv_decode_opts* opts,
                                 int32_t num_seqs, const int8_t* q_int8, const float* q_scale,
                                 const int8_t* k_cache, const int8_t* v_cache,
                                 const float* k_scale, const float* v_scale,
                                 const int32_t* block_tables, int32_t max_blocks_per_seq,
                                 const int32_t* seq_lens, int32_t max_seq_len, void* workspace,
                                 size_t workspace_bytes, void* out, i8kv_stream_t stream);

/*
 * One decode step with the producer fused in: for every sequence s, the
 * newest token (position seq_lens[s] - 1) is quantized and written to the
 * cache as i8kv_kv_quantize_write would write it ([KV] 2.1-2.3, with its slot
 * taken from block_tables), its query is quantized once ([KV] 2.2), and the
 * token's query attends to all seq_lens[s] tokens exactly as
 * i8kv_paged_decode_int8 computes it ([KV] 3.3; [PV] 2.2).  Caches, scales,
 * q_int8 / q_scale and out are bit-identical to those two calls in sequence;
 * the step is one partition kernel (plus the merge kernel) instead of three
 * kernels.
 *   key, value   [S, Hkv, D] bf16      query [S, Hq, D] bf16 (the newest tokens)
 *   q_int8 [S, Hq, D], q_scale [S, Hq]: optional outputs (both NULL or both set)
 *   caches as for i8kv_kv_quantize_write; the page of position seq_lens[s] - 1
 *   is block_tables[s][(seq_lens[s] - 1) / 16] (an entry outside [0, num_blocks)
 *   skips the write, as a negative slot does for the producer); a sequence
 *   with seq_lens[s] = 0 writes no token and outputs zeros.
 *   Other arguments, workspace and errors as for i8kv_paged_decode_int8
 *   (NULL also for a missing key/value/query or only one of q_int8/q_scale).
 */
i8kv_status i8kv_decode_step_int8(const i8kv_cache_desc* desc, int32_t num_seqs,
                                  const uint16_t* key, const uint16_t* value,
                                  const uint16_t* query, int8_t* q_int8, float* q_scale,
                                  int8_t* k_cache, int8_t* v_cache, float* k_scale,
                                  float* v_scale, const int32_t* block_tables,
                                  int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                  int32_t max_seq_len, int32_t partition_size, int32_t w_group,
                                  float softmax_scale, void* workspace, size_t workspace_bytes,
                                  float* out, i8kv_stream_t stream);

/* Workspace bytes for i8kv_prefix_prefill_int8, for the memory budget of
 * [KV] 5.6.  The prefill keeps its (m, l, o) state on chip, so this is 0. */
size_t i8kv_prefix_prefill_workspace_bytes(const i8kv_cache_desc* desc, int32_t num_seqs,
                                           int32_t total_q);

/*
 * Chunked prefill with history ([KV] 3.2; [PV] 2.1).  Sequence s owns query
 * rows query_start_loc[s] .. query_start_loc[s+1]-1 (its chunk of
 * c_s tokens); the chunk's own K/V must already be in the cache (written by
 * the producer), so seq_lens[s] counts history + chunk.  Row j of the chunk
 * sits at absolute position seq_lens[s] - c_s + j and sees keys 0..position
 * (causal within the chunk).  History and chunk go through ONE online softmax:
 *   m' = max(m, max s), alpha = exp(m - m'), p~_i = exp(s_i - m'),
 *   W_i = p~_i * sV_i, group-quantized per aligned w_group keys as in decode,
 *   o = alpha o + sum_g sW (Wq x Vq), l = alpha l + sum p~_i, O = o / l.
 *   q_int8 [total_q, Hq, D], q_scale [total_q, Hq]
 *   query_start_loc [S+1] int32, seq_lens [S] int32,
 *   block_tables [S, max_blocks_per_seq] int32
 *   max_query_len >= every chunk length (sizes the launch grid)
 *   out [total_q, Hq, D] fp32, fully overwritten.
 * Numerics: fp32; the codes use a hardware reciprocal of max W (a code may
 * differ by one on a near-tie of W / sW) and, for w_group 32, the dequantizing
 * sW is cut to 22 significant bits (relative change < 2^-21), so outputs
 * follow the definition to rounding, not bit for bit.
 * Errors: NULL, INVALID_ARG, UNSUPPORTED (as for decode), WORKSPACE.
 */
i8kv_status i8kv_prefix_prefill_int8(const i8kv_cache_desc* desc, int32_t num_seqs,
                                     int32_t total_q, int32_t max_query_len,
                                     const int8_t* q_int8, const float* q_scale,
                                     const int32_t* query_start_loc,
                                     const int32_t* seq_lens, const int8_t* k_cache,
                                     const int8_t* v_cache, const float* k_scale,
                                     const float* v_scale, const int32_t* block_tables,
                                     int32_t max_blocks_per_seq, int32_t w_group,
                                     float softmax_scale, void* workspace,
                                     size_t workspace_bytes, float* out,
                                     i8kv_stream_t stream);

/*
 * The UINT8-W variant of i8kv_prefix_prefill_int8 ([PV] 6: W = p~ sV >= 0, so
 * unsigned codes give one more bit): per aligned group of w_group keys
 *   sW = max W / 255 (IEEE), Wq = round(W / sW) in [0, 255] (half away from
 *   zero on the definition's division; the kernel's reciprocal rule may move a
 *   code by one on a near-tie), o = alpha o + sum_g sW (Wq x Vq);
 * everything else as i8kv_prefix_prefill_int8.  gfx950's int8 MFMA is signed,
 * so the codes enter it as Wq - 128 and a second MFMA against all-ones rows
 * returns the group's sum of Vq, of which 128 times is added back in int32
 * (exact).  Arguments and errors as for i8kv_prefix_prefill_int8.
 */
i8kv_status i8kv_prefix_prefill_uint8w(const i8kv_cache_desc* desc, int32_t num_seqs,
                                       int32_t total_q, int32_t max_query_len,
                                       const int8_t* q_int8, const float* q_scale,
                                       const int32_t* query_start_loc, const int32_t* seq_lens,
                                       const int8_t* k_cache, const int8_t* v_cache,
                                       const float* k_scale, const float* v_scale,
                                       const int32_t* block_tables, int32_t max_blocks_per_seq,
                                       int32_t w_group, float softmax_scale, void* workspace,
                                       size_t workspace_bytes, float* out,
                                       i8kv_stream_t stream);

/*
 * The prefill with options, in the serving shape of the pages' attention
 * call ([KV] 3.2 outputs bf16):
 *  - pv: the method's int8 W groups (I8KV_PV_INT8), the BF16-PV ablation
 *    (I8KV_PV_BF16, w_group unused) or UINT8 W (I8KV_PV_UINT8) -- the
 *    computations of i8kv_prefix_prefill_int8, _bf16pv and _uint8w;
 *  - out_bf16: out [total_q, Hq, D] holds the fp32 result rounded to bf16
 *    (nearest, ties to even; 8-byte aligned) instead of fp32.
 * Other arguments as for i8kv_prefix_prefill_int8 (no workspace).
 * Errors: as i8kv_prefix_prefill_int8; NULL for opts; INVALID_ARG for
 * out_bf16 not 0/1 or a misaligned bf16 out; UNSUPPORTED for an unknown pv.
 */
typedef struct {
  int32_t w_group;      /* 32 or 64 (unused by I8KV_PV_BF16) */
  float softmax_scale;
  int32_t pv;           /* I8KV_PV_INT8 (the method), _BF16 or _UINT8 */
  int32_t out_bf16;     /* 0: out is fp32; 1: out is bf16 bits */
} i8kv_prefill_opts;

i8kv_status i8kv_prefix_prefill_ex(const i8kv_cache_desc* desc, const i8kv_prefill_opts* opts,
                                   int32_t num_seqs, int32_t total_q, int32_t max_query_len,
                                   const int8_t* q_int8, const float* q_scale,
                                   const int32_t* query_start_loc, const int32_t* seq_lens,
                                   const int8_t* k_cache, const int8_t* v_cache,
                                   const float* k_scale, const float* v_scale,
                                   const int32_t* block_tables, int32_t max_blocks_per_seq,
                                   void* out, i8kv_stream_t stream);

/*
 * The BF16-PV ablation of i8kv_prefix_prefill_int8 ([PV] 5): the same scores
 * and online softmax, but W = p~ * sV is rounded to bf16 (nearest, ties to
 * even) instead of group-quantized, and o = alpha o + sum_i bf16(W_i) Vq_i
 * with the int8 V taken exactly as bf16 and fp32 accumulation
 * (v_mfma_f32_16x16x32_bf16); the output is rescaled whenever the running
 * maximum grows (64-key tiles).  Arguments and errors as
 * i8kv_prefix_prefill_int8 without w_group.
 */
i8kv_status i8kv_prefix_prefill_bf16pv(const i8kv_cache_desc* desc, int32_t num_seqs,
                                       int32_t total_q, int32_t max_query_len,
                                       const int8_t* q_int8, const float* q_scale,
                                       const int32_t* query_start_loc, const int32_t* seq_lens,
                                       const int8_t* k_cache, const int8_t* v_cache,
                                       const float* k_scale, const float* v_scale,
                                       const int32_t* block_tables, int32_t max_blocks_per_seq,
                                       float softmax_scale, void* workspace,
                                       size_t workspace_bytes, float* out,
                                       i8kv_stream_t stream);

/*
 * The BF16-QK ablation of i8kv_prefix_prefill_int8 ([KV] 4.1): the queries
 * are not quantized; each landed K tile is converted to bf16 (exact for int8
 * codes) and S = Q K^T runs on v_mfma_f32_16x16x32_bf16 with fp32
 * accumulation, score = (dot * sK) * softmax_scale.  The online softmax, the
 * int8 W groups and the PV product are those of i8kv_prefix_prefill_int8
 * (workgroups of 128 flattened rows instead of 192).
 *   query_bf16 [total_q, Hq, D] bf16 bits (16-byte aligned) in place of
 *   q_int8 and q_scale; every other argument and the errors as
 *   i8kv_prefix_prefill_int8.
 */
i8kv_status i8kv_prefix_prefill_bf16qk(const i8kv_cache_desc* desc, int32_t num_seqs,
                                       int32_t total_q, int32_t max_query_len,
                                       const uint16_t* query_bf16,
                                       const int32_t* query_start_loc, const int32_t* seq_lens,
                                       const int8_t* k_cache, const int8_t* v_cache,
                                       const float* k_scale, const float* v_scale,
                                       const int32_t* block_tables, int32_t max_blocks_per_seq,
                                       int32_t w_group, float softmax_scale, void* workspace,
                                       size_t workspace_bytes, float* out,
                                       i8kv_stream_t stream);

/* Human-readable name of a status code (static string); any other value
 * gives "unknown status".  Takes the code as an int32_t so that a value no
 * i8kv_status names is still a valid argument. */
const char* i8kv_status_string(int32_t status);

/* I8KV_ABI_VERSION of the loaded library. */
int32_t i8kv_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* I8KV_H */
