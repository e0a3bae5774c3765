// Internal launch interface between the C ABI (abi.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace i8kv {

constexpr int kBlockSize = 16;   // tokens per page
constexpr int kPartition = 256;  // decode partition (tokens)

struct ProducerArgs {
  int32_t num_tokens, num_q_heads, num_kv_heads, head_dim, num_blocks;
  const uint16_t* key;
  const uint16_t* value;
  const uint16_t* query;  // may be null
  int8_t* q_int8;
  float* q_scale;
  const int32_t* slot_mapping;
  int8_t* k_cache;
  int8_t* v_cache;
  float* k_scale;
  float* v_scale;
  // Rotary embedding of Q and K (positions == null: none).
  const int32_t* positions;  // [T]
  const float* cos_sin;      // [max_position, rotary_dim]: cos | sin
  int32_t rotary_dim, max_position;
};

hipError_t launch_kv_quantize_write(const ProducerArgs& a, hipStream_t stream);

// Decode workspace: per-partition partial outputs and (m, l).
struct DecodePlan {
  int32_t num_seqs, num_kv_heads, group;  // group = Hq / Hkv
  int32_t head_dim;
  int32_t max_parts;    // ceil(max_seq_len / 256)
  size_t off_part_o, off_part_ml, bytes;
};

DecodePlan make_decode_plan(int32_t num_seqs, int32_t num_kv_heads, int32_t group,
                            int32_t head_dim, int32_t max_seq_len);

struct DecodeArgs {
  int32_t num_seqs, num_q_heads, num_kv_heads, group, head_dim, num_blocks;
  int32_t max_blocks_per_seq, max_seq_len, w_group;
  int32_t pv_bf16;  // the BF16-PV ablation (w_group unused)
  int32_t w_uint8;  // UINT8 W groups (codes 0..255, sW = max W / 255)
  int32_t nq;       // queries per sequence (the newest nq positions, causal)
  float softmax_scale;
  const int8_t* q_int8;
  const float* q_scale;
  const uint16_t* q_bf16;  // the BF16-QK ablation: bf16 queries [S, Hq, D] instead
  const int8_t* k_cache;
  const int8_t* v_cache;
  const float* k_scale;
  const float* v_scale;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  float* out;
  uint16_t* out16;  // bf16 output instead of out (nearest, ties to even)
  // fused step (producer of each sequence's newest token + decode); new_key is
  // null for a plain decode
  const uint16_t* new_key;    // [S, Hkv, D] bf16
  const uint16_t* new_value;  // [S, Hkv, D] bf16
  const uint16_t* new_query;  // [S, Hq, D] bf16
  int8_t* k_cache_w;          // the caches, written at position seq_lens[s] - 1
  int8_t* v_cache_w;
  float* k_scale_w;
  float* v_scale_w;
  int8_t* q_int8_w;           // optional Q outputs [S, Hq, D], [S, Hq]
  float* q_scale_w;
  // workspace views
  float* part_o;    // [S, Hkv, max_parts, group, D]
  float* part_ml;   // [S, Hkv, max_parts, group, 2]
  int32_t max_parts;
  // The two stages run alone: 1 = partitions only (every sequence's partials
  // go to the workspace, single-partition ones included, nothing to `out`);
  // 2 = merge only (every sequence, single-partition and empty ones
  // included, from the workspace to `out`); 0 = both, as one call.
  int32_t stage;
};

hipError_t launch_paged_decode(const DecodeArgs& a, hipStream_t stream);

struct PrefillArgs {
  int32_t num_seqs, total_q, max_query_len, num_q_heads, num_kv_heads, group, head_dim,
      num_blocks, max_blocks_per_seq, w_group;
  int32_t pv_bf16;  // the BF16-PV ablation (w_group unused)
  int32_t w_uint8;  // UINT8 W groups (codes 0..255, sW = max W / 255)
  float softmax_scale;
  const int8_t* q_int8;
  const float* q_scale;
  const uint16_t* q_bf16;  // the BF16-QK ablation: bf16 queries [Tq, Hq, D] instead
  const int32_t* query_start_loc;
  const int32_t* seq_lens;
  const int8_t* k_cache;
  const int8_t* v_cache;
  const float* k_scale;
  const float* v_scale;
  const int32_t* block_tables;
  float* out;
  uint16_t* out16;  // bf16 output instead of out (nearest, ties to even)
};

hipError_t launch_prefix_prefill(const PrefillArgs& a, hipStream_t stream);

}  // namespace i8kv
