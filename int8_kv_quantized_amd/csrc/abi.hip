// C ABI of libi8kv: argument validation on the host, then one launch.
// Every check below runs before anything is enqueued; no exception crosses
// the ABI.  The declarations and their documentation are in include/i8kv.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>

#include "i8kv.h"
#include "kernels.hpp"

namespace {

using namespace i8kv;

constexpr int32_t kMaxSeqLen = 1 << 20;  // at most 4096 decode partitions
constexpr int32_t kMaxGridYZ = 65535;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

i8kv_status check_desc(const i8kv_cache_desc* d) {
  if (!d) return I8KV_ERR_NULL;
  if (d->num_q_heads <= 0 || d->num_kv_heads <= 0 || d->head_dim <= 0 || d->num_blocks <= 0 ||
      d->block_size <= 0)
    return I8KV_ERR_INVALID_ARG;
  if (d->block_size != kBlockSize) return I8KV_ERR_UNSUPPORTED;
  if (d->head_dim != 64 && d->head_dim != 128 && d->head_dim != 256) return I8KV_ERR_UNSUPPORTED;
  if (d->num_q_heads % d->num_kv_heads != 0) return I8KV_ERR_UNSUPPORTED;
  if (d->num_q_heads / d->num_kv_heads > 16) return I8KV_ERR_UNSUPPORTED;
  if (d->num_kv_heads > kMaxGridYZ) return I8KV_ERR_UNSUPPORTED;
  return I8KV_OK;
}

i8kv_status from_hip(hipError_t e) { return e == hipSuccess ? I8KV_OK : I8KV_ERR_LAUNCH; }

// The launch wrappers report hipGetLastError() after enqueuing, which also
// returns an error left behind by any earlier runtime call of the calling
// thread (not necessarily one of ours).  Each entry point therefore clears that
// pending, non-sticky error right before it launches, so the status it returns
// describes its own launches; a sticky error (a device fault) persists and is
// still reported.
hipError_t launch_clean(hipError_t (*launch)(const ProducerArgs&, hipStream_t),
                        const ProducerArgs& a, hipStream_t st) {
  (void)hipGetLastError();
  return launch(a, st);
}
hipError_t launch_clean(hipError_t (*launch)(const PrefillArgs&, hipStream_t),
                        const PrefillArgs& a, hipStream_t st) {
  (void)hipGetLastError();
  return launch(a, st);
}
hipError_t launch_clean(hipError_t (*launch)(const DecodeArgs&, hipStream_t),
                        const DecodeArgs& a, hipStream_t st) {
  (void)hipGetLastError();
  return launch(a, st);
}

// Shared by the producer entry points; positions == null means no rotation.
i8kv_status run_producer(const i8kv_cache_desc* desc, int32_t num_tokens, const uint16_t* key,
                         const uint16_t* value, const uint16_t* query, int8_t* q_int8,
                         float* q_scale, const int32_t* slot_mapping, const int32_t* positions,
                         const float* cos_sin, int32_t rotary_dim, int32_t max_position,
                         int8_t* k_cache, int8_t* v_cache, float* k_scale, float* v_scale,
                         i8kv_stream_t stream) {
  i8kv_status st = check_desc(desc);
  if (st != I8KV_OK) return st;
  if (!key || !value || !slot_mapping || !k_cache || !v_cache || !k_scale || !v_scale)
    return I8KV_ERR_NULL;
  if (query && (!q_int8 || !q_scale)) return I8KV_ERR_NULL;
  if (num_tokens < 0) return I8KV_ERR_INVALID_ARG;
  if (!aligned16(key) || !aligned16(value) || (query && (!aligned16(query) || !aligned16(q_int8))) ||
      !aligned16(k_cache) || !aligned16(v_cache))
    return I8KV_ERR_INVALID_ARG;
  if (positions) {
    if (max_position <= 0 || rotary_dim <= 0 || (reinterpret_cast<uintptr_t>(cos_sin) & 3u))
      return I8KV_ERR_INVALID_ARG;
    const int per_lane = desc->head_dim / 64;
    if (rotary_dim > desc->head_dim || rotary_dim % (2 * per_lane) != 0)
      return I8KV_ERR_UNSUPPORTED;
  }
  if (num_tokens == 0) return I8KV_OK;
  ProducerArgs a{};
  a.num_tokens = num_tokens;
  a.num_q_heads = desc->num_q_heads;
  a.num_kv_heads = desc->num_kv_heads;
  a.head_dim = desc->head_dim;
  a.num_blocks = desc->num_blocks;
  a.key = key;
  a.value = value;
  a.query = query;
  a.q_int8 = q_int8;
  a.q_scale = q_scale;
  a.slot_mapping = slot_mapping;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.positions = positions;
  a.cos_sin = cos_sin;
  a.rotary_dim = rotary_dim;
  a.max_position = max_position;
  return from_hip(launch_clean(launch_kv_quantize_write, a, static_cast<hipStream_t>(stream)));
}

}  // namespace

namespace {

i8kv_status run_prefill(const i8kv_cache_desc* desc, int32_t num_seqs,
                                     int32_t total_q, int32_t max_query_len,
                                     const int8_t* q_int8, const float* q_scale,
                                     const int32_t* query_start_loc, const int32_t* seq_lens,
                                     const int8_t* k_cache, const int8_t* v_cache,
                                     const float* k_scale, const float* v_scale,
                                     const int32_t* block_tables, int32_t max_blocks_per_seq,
                                     int32_t w_group, float softmax_scale, void* workspace,
                                     size_t workspace_bytes, float* out,
                                     i8kv_stream_t stream, bool pv_bf16,
                                     const uint16_t* q_bf16 = nullptr, bool w_uint8 = false,
                                     uint16_t* out16 = nullptr) {
  (void)workspace;
  (void)workspace_bytes;
  i8kv_status st = check_desc(desc);
  if (st != I8KV_OK) return st;
  if ((!q_bf16 && (!q_int8 || !q_scale)) || !query_start_loc || !seq_lens || !k_cache ||
      !v_cache || !k_scale || !v_scale || !block_tables || (!out && !out16))
    return I8KV_ERR_NULL;
  if (num_seqs < 0 || total_q < 0 || max_query_len < 0 || max_blocks_per_seq <= 0)
    return I8KV_ERR_INVALID_ARG;
  if (max_query_len > total_q) return I8KV_ERR_INVALID_ARG;
  if (!std::isfinite(softmax_scale)) return I8KV_ERR_INVALID_ARG;
  if (w_group != 32 && w_group != 64) return I8KV_ERR_UNSUPPORTED;
  if (num_seqs > kMaxGridYZ) return I8KV_ERR_UNSUPPORTED;
  if ((q_bf16 ? !aligned16(q_bf16) : !aligned16(q_int8)) || !aligned16(k_cache) ||
      !aligned16(v_cache))
    return I8KV_ERR_INVALID_ARG;
  if (out16 && (reinterpret_cast<uintptr_t>(out16) & 7)) return I8KV_ERR_INVALID_ARG;
  if (num_seqs == 0 || total_q == 0) return I8KV_OK;
  PrefillArgs a{};
  a.num_seqs = num_seqs;
  a.total_q = total_q;
  a.max_query_len = max_query_len;
  a.num_q_heads = desc->num_q_heads;
  a.num_kv_heads = desc->num_kv_heads;
  a.group = desc->num_q_heads / desc->num_kv_heads;
  a.head_dim = desc->head_dim;
  a.num_blocks = desc->num_blocks;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.w_group = w_group;
  a.pv_bf16 = pv_bf16 ? 1 : 0;
  a.w_uint8 = w_uint8 ? 1 : 0;
  a.softmax_scale = softmax_scale;
  a.q_int8 = q_bf16 ? nullptr : q_int8;
  a.q_scale = q_bf16 ? nullptr : q_scale;
  a.q_bf16 = q_bf16;
  a.query_start_loc = query_start_loc;
  a.seq_lens = seq_lens;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.block_tables = block_tables;
  a.out = out16 ? nullptr : out;
  a.out16 = out16;
  return from_hip(launch_clean(launch_prefix_prefill, a, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

int32_t i8kv_abi_version(void) { return I8KV_ABI_VERSION; }

const char* i8kv_status_string(int32_t s) {
  switch (s) {
    case I8KV_OK: return "ok";
    case I8KV_ERR_NULL: return "null pointer argument";
    case I8KV_ERR_INVALID_ARG: return "invalid argument";
    case I8KV_ERR_UNSUPPORTED: return "unsupported shape or parameter";
    case I8KV_ERR_WORKSPACE: return "workspace missing or too small";
    case I8KV_ERR_LAUNCH: return "kernel launch failed";
  }
  return "unknown status";
}

i8kv_status i8kv_kv_quantize_write(const i8kv_cache_desc* desc, int32_t num_tokens,
                                   const uint16_t* key, const uint16_t* value,
                                   const uint16_t* query, int8_t* q_int8, float* q_scale,
                                   const int32_t* slot_mapping, int8_t* k_cache,
                                   int8_t* v_cache, float* k_scale, float* v_scale,
                                   i8kv_stream_t stream) {
  return run_producer(desc, num_tokens, key, value, query, q_int8, q_scale, slot_mapping,
                      nullptr, nullptr, 0, 0, k_cache, v_cache, k_scale, v_scale, stream);
}

i8kv_status i8kv_kv_quantize_write_rope(const i8kv_cache_desc* desc, int32_t num_tokens,
                                        const uint16_t* key, const uint16_t* value,
                                        const uint16_t* query, int8_t* q_int8, float* q_scale,
                                        const int32_t* slot_mapping, const int32_t* positions,
                                        const float* cos_sin, int32_t rotary_dim,
                                        int32_t max_position, int8_t* k_cache, int8_t* v_cache,
                                        float* k_scale, float* v_scale, i8kv_stream_t stream) {
  if (!positions || !cos_sin) return I8KV_ERR_NULL;
  return run_producer(desc, num_tokens, key, value, query, q_int8, q_scale, slot_mapping,
                      positions, cos_sin, rotary_dim, max_position, k_cache, v_cache, k_scale,
                      v_scale, stream);
}

size_t i8kv_paged_decode_workspace_bytes(const i8kv_cache_desc* desc, int32_t num_seqs,
                                         int32_t max_seq_len, int32_t partition_size) {
  if (check_desc(desc) != I8KV_OK || num_seqs < 0 || max_seq_len < 0 ||
      max_seq_len > kMaxSeqLen || partition_size != kPartition)
    return 0;
  const DecodePlan p = make_decode_plan(num_seqs, desc->num_kv_heads,
                                        desc->num_q_heads / desc->num_kv_heads,
                                        desc->head_dim, max_seq_len);
  return p.bytes;
}

}  // extern "C"

namespace {

// Shared by the decode and the fused decode-step entry points: validation and
// argument packing, then the launch.  `fused` carries the producer inputs and
// outputs of the step (new_key non-null), with q_int8 / q_scale then optional
// outputs rather than inputs.
i8kv_status run_decode(const i8kv_cache_desc* desc, int32_t num_seqs, const int8_t* q_int8,
                       const float* q_scale, const int8_t* k_cache, const int8_t* v_cache,
                       const float* k_scale, const float* v_scale, const int32_t* block_tables,
                       int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t max_seq_len,
                       int32_t partition_size, int32_t w_group, float softmax_scale,
                       void* workspace, size_t workspace_bytes, float* out,
                       const DecodeArgs* fused, i8kv_stream_t stream, bool pv_bf16 = false,
                       bool w_uint8 = false, int32_t nq = 1, uint16_t* out16 = nullptr,
                       const uint16_t* q_bf16 = nullptr, int32_t stage = 0) {
  i8kv_status st = check_desc(desc);
  if (st != I8KV_OK) return st;
  // stage 1 (partitions alone) has no output; stage 2 (merge alone) reads only
  // the sequence lengths and the workspace
  if (!seq_lens || (stage != 1 && !out && !out16)) return I8KV_ERR_NULL;
  if (stage != 2 && (!k_cache || !v_cache || !k_scale || !v_scale || !block_tables))
    return I8KV_ERR_NULL;
  if (stage != 2 && !fused && !q_bf16 && (!q_int8 || !q_scale)) return I8KV_ERR_NULL;
  if (fused && (!fused->new_key || !fused->new_value || !fused->new_query)) return I8KV_ERR_NULL;
  if (fused && (!q_int8) != (!q_scale)) return I8KV_ERR_NULL;
  if (num_seqs < 0 || max_seq_len < 0 || max_blocks_per_seq <= 0) return I8KV_ERR_INVALID_ARG;
  if ((int64_t)max_seq_len > (int64_t)max_blocks_per_seq * kBlockSize) return I8KV_ERR_INVALID_ARG;
  if (!std::isfinite(softmax_scale)) return I8KV_ERR_INVALID_ARG;
  if (partition_size != kPartition || (w_group != 32 && w_group != 64))
    return I8KV_ERR_UNSUPPORTED;
  if (nq < 1) return I8KV_ERR_INVALID_ARG;
  if ((int64_t)nq * (desc->num_q_heads / desc->num_kv_heads) > 16 || (fused && nq != 1) ||
      (int64_t)nq * desc->num_q_heads > 0x7fffffff)
    return I8KV_ERR_UNSUPPORTED;
  if (max_seq_len > kMaxSeqLen || num_seqs > kMaxGridYZ) return I8KV_ERR_UNSUPPORTED;
  if ((q_int8 && !aligned16(q_int8)) || (q_bf16 && !aligned16(q_bf16)) ||
      (k_cache && !aligned16(k_cache)) || (v_cache && !aligned16(v_cache)) ||
      (out && !aligned16(out)) || (out16 && !aligned16(out16)))
    return I8KV_ERR_INVALID_ARG;
  if (fused && (!aligned16(fused->new_key) || !aligned16(fused->new_value) ||
                !aligned16(fused->new_query)))
    return I8KV_ERR_INVALID_ARG;
  if (num_seqs == 0) return I8KV_OK;
  const int32_t grp = desc->num_q_heads / desc->num_kv_heads;
  const DecodePlan p =
      make_decode_plan(num_seqs, desc->num_kv_heads, grp * nq, desc->head_dim, max_seq_len);
  if (!workspace || workspace_bytes < p.bytes) return I8KV_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return I8KV_ERR_WORKSPACE;

  char* ws = static_cast<char*>(workspace);
  DecodeArgs a{};
  if (fused) a = *fused;  // producer pointers of the fused step
  a.num_seqs = num_seqs;
  a.num_q_heads = desc->num_q_heads;
  a.num_kv_heads = desc->num_kv_heads;
  a.group = grp;
  a.head_dim = desc->head_dim;
  a.num_blocks = desc->num_blocks;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.max_seq_len = max_seq_len;
  a.w_group = w_group;
  a.pv_bf16 = pv_bf16 ? 1 : 0;
  a.w_uint8 = w_uint8 ? 1 : 0;
  a.nq = nq;
  a.softmax_scale = softmax_scale;
  a.q_int8 = fused || q_bf16 ? nullptr : q_int8;
  a.q_scale = fused || q_bf16 ? nullptr : q_scale;
  a.q_bf16 = fused ? nullptr : q_bf16;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.block_tables = block_tables;
  a.seq_lens = seq_lens;
  a.out = out16 ? nullptr : out;
  a.out16 = out16;
  a.part_o = reinterpret_cast<float*>(ws + p.off_part_o);
  a.part_ml = reinterpret_cast<float*>(ws + p.off_part_ml);
  a.max_parts = p.max_parts;
  a.stage = stage;
  return from_hip(launch_clean(launch_paged_decode, a, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

i8kv_status i8kv_paged_decode_int8(const i8kv_cache_desc* desc, int32_t num_seqs,
                                   const int8_t* q_int8, const float* q_scale,
                                   const int8_t* k_cache, const int8_t* v_cache,
                                   const float* k_scale, const float* v_scale,
                                   const int32_t* block_tables, int32_t max_blocks_per_seq,
                                   const int32_t* seq_lens, int32_t max_seq_len,
                                   int32_t partition_size, int32_t w_group,
                                   float softmax_scale, void* workspace,
                                   size_t workspace_bytes, float* out,
                                   i8kv_stream_t stream) {
  return run_decode(desc, num_seqs, q_int8, q_scale, k_cache, v_cache, k_scale, v_scale,
                    block_tables, max_blocks_per_seq, seq_lens, max_seq_len, partition_size,
                    w_group, softmax_scale, workspace, workspace_bytes, out, nullptr, stream);
}

i8kv_status i8kv_paged_decode_partials(const i8kv_cache_desc* desc, int32_t num_seqs,
                                       const int8_t* q_int8, const float* q_scale,
                                       const int8_t* k_cache, const int8_t* v_cache,
                                       const float* k_scale, const float* v_scale,
                                       const int32_t* block_tables, int32_t max_blocks_per_seq,
                                       const int32_t* seq_lens, int32_t max_seq_len,
                                       int32_t partition_size, int32_t w_group,
                                       float softmax_scale, void* workspace,
                                       size_t workspace_bytes, i8kv_stream_t stream) {
  return run_decode(desc, num_seqs, q_int8, q_scale, k_cache, v_cache, k_scale, v_scale,
                    block_tables, max_blocks_per_seq, seq_lens, max_seq_len, partition_size,
                    w_group, softmax_scale, workspace, workspace_bytes, nullptr, nullptr, stream,
                    false, false, 1, nullptr, nullptr, /*stage=*/1);
}

i8kv_status i8kv_paged_decode_merge(const i8kv_cache_desc* desc, int32_t num_seqs,
                                    const int32_t* seq_lens, int32_t max_seq_len,
                                    int32_t partition_size, const void* workspace,
                                    size_t workspace_bytes, float* out, i8kv_stream_t stream) {
  // the merge reads no page: a table width that admits max_seq_len, no cache
  const int32_t width = max_seq_len > 0 ? (max_seq_len + kBlockSize - 1) / kBlockSize : 1;
  return run_decode(desc, num_seqs, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                    nullptr, width, seq_lens, max_seq_len, partition_size, 32, 1.0f,
                    const_cast<void*>(workspace), workspace_bytes, out, nullptr, stream, false,
                    false, 1, nullptr, nullptr, /*stage=*/2);
}

i8kv_status i8kv_paged_decode_bf16pv(const i8kv_cache_desc* desc, int32_t num_seqs,
                                     const int8_t* q_int8, const float* q_scale,
                                     const int8_t* k_cache, const int8_t* v_cache,
                                     const float* k_scale, const float* v_scale,
                                     const int32_t* block_tables, int32_t max_blocks_per_seq,
                                     const int32_t* seq_lens, int32_t max_seq_len,
                                     int32_t partition_size, float softmax_scale, void* workspace,
                                     size_t workspace_bytes, float* out, i8kv_stream_t stream) {
  return run_decode(desc, num_seqs, q_int8, q_scale, k_cache, v_cache, k_scale, v_scale,
                    block_tables, max_blocks_per_seq, seq_lens, max_seq_len, partition_size,
                    64, softmax_scale, workspace, workspace_bytes, out, nullptr, stream,
                    /*pv_bf16=*/true);
}

i8kv_status i8kv_paged_decode_uint8w(const i8kv_cache_desc* desc, int32_t num_seqs,
                                     const int8_t* q_int8, const float* q_scale,
                                     const int8_t* k_cache, const int8_t* v_cache,
                                     const float* k_scale, const float* v_scale,
                                     const int32_t* block_tables, int32_t max_blocks_per_seq,
                                     const int32_t* seq_lens, int32_t max_seq_len,
                                     int32_t partition_size, int32_t w_group,
                                     float softmax_scale, void* workspace,
                                     size_t workspace_bytes, float* out, i8kv_stream_t stream) {
  return run_decode(desc, num_seqs, q_int8, q_scale, k_cache, v_cache, k_scale, v_scale,
                    block_tables, max_blocks_per_seq, seq_lens, max_seq_len, partition_size,
                    w_group, softmax_scale, workspace, workspace_bytes, out, nullptr, stream,
                    /*pv_bf16=*/false, /*w_uint8=*/true);
}

i8kv_status i8kv_paged_decode_bf16qk(const i8kv_cache_desc* desc, int32_t num_seqs,
                                     const uint16_t* query_bf16, const int8_t* k_cache,
                                     const int8_t* v_cache, const float* k_scale,
                                     const float* v_scale, const int32_t* block_tables,
                                     int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                     int32_t max_seq_len, int32_t partition_size,
                                     int32_t w_group, float softmax_scale, void* workspace,
                                     size_t workspace_bytes, float* out, i8kv_stream_t stream) {
  if (!query_bf16) return I8KV_ERR_NULL;
  return run_decode(desc, num_seqs, nullptr, nullptr, k_cache, v_cache, k_scale, v_scale,
                    block_tables, max_blocks_per_seq, seq_lens, max_seq_len, partition_size,
                    w_group, softmax_scale, workspace, workspace_bytes, out, nullptr, stream,
                    /*pv_bf16=*/false, /*w_uint8=*/false, /*nq=*/1, /*out16=*/nullptr, query_bf16);
}

size_t i8kv_paged_decode_ex_workspace_bytes(const i8kv_cache_desc* desc,
                                            const i8kv_decode_opts* opts, int32_t num_seqs,
                                            int32_t max_seq_len) {
  if (!opts || check_desc(desc) != I8KV_OK || num_seqs < 0 || max_seq_len < 0 ||
      max_seq_len > kMaxSeqLen || opts->partition_size != kPartition ||
      opts->queries_per_seq < 1 || opts->queries_per_seq > 16)
    return 0;
  const DecodePlan p = make_decode_plan(
      num_seqs, desc->num_kv_heads,
      desc->num_q_heads / desc->num_kv_heads * opts->queries_per_seq, desc->head_dim, max_seq_len);
  return p.bytes;
}

i8kv_status i8kv_paged_decode_ex(const i8kv_cache_desc* desc, const i8kv_decode_opts* opts,
                                 int32_t num_seqs, const int8_t* q_int8, const float* q_scale,
                                 const int8_t* k_cache, const int8_t* v_cache,
                                 const float* k_scale, const float* v_scale,
                                 const int32_t* block_tables, int32_t max_blocks_per_seq,
                                 const int32_t* seq_lens, int32_t max_seq_len, void* workspace,
                                 size_t workspace_bytes, void* out, i8kv_stream_t stream) {
  if (!opts) return I8KV_ERR_NULL;
  if (opts->pv != I8KV_PV_INT8 && opts->pv != I8KV_PV_BF16 && opts->pv != I8KV_PV_UINT8)
    return I8KV_ERR_UNSUPPORTED;
  if (opts->out_bf16 != 0 && opts->out_bf16 != 1) return I8KV_ERR_INVALID_ARG;
  const bool bf16 = opts->pv == I8KV_PV_BF16;
  return run_decode(desc, num_seqs, q_int8, q_scale, k_cache, v_cache, k_scale, v_scale,
                    block_tables, max_blocks_per_seq, seq_lens, max_seq_len,
                    opts->partition_size, bf16 ? 64 : opts->w_group, opts->softmax_scale,
                    workspace, workspace_bytes, opts->out_bf16 ? nullptr : static_cast<float*>(out),
                    nullptr, stream, bf16, opts->pv == I8KV_PV_UINT8, opts->queries_per_seq,
                    opts->out_bf16 ? static_cast<uint16_t*>(out) : nullptr);
}

i8kv_status i8kv_decode_step_int8(const i8kv_cache_desc* desc, int32_t num_seqs,
                                  const uint16_t* key, const uint16_t* value,
                                  const uint16_t* query, int8_t* q_int8, float* q_scale,
                                  int8_t* k_cache, int8_t* v_cache, float* k_scale,
                                  float* v_scale, const int32_t* block_tables,
                                  int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                  int32_t max_seq_len, int32_t partition_size, int32_t w_group,
                                  float softmax_scale, void* workspace, size_t workspace_bytes,
                                  float* out, i8kv_stream_t stream) {
  DecodeArgs f{};
  f.new_key = key;
  f.new_value = value;
  f.new_query = query;
  f.k_cache_w = k_cache;
  f.v_cache_w = v_cache;
  f.k_scale_w = k_scale;
  f.v_scale_w = v_scale;
  f.q_int8_w = q_int8;
  f.q_scale_w = q_scale;
  return run_decode(desc, num_seqs, q_int8, q_scale, k_cache, v_cache, k_scale, v_scale,
                    block_tables, max_blocks_per_seq, seq_lens, max_seq_len, partition_size,
                    w_group, softmax_scale, workspace, workspace_bytes, out, &f, stream);
}

}  // extern "C"

namespace {

// ---- the decode for callers that cannot allocate ---------------------------
// Partials of i8kv_paged_decode_int8_noalloc: a fixed device array, one copy
// per GPU, alive until the process ends.  In host code `scratch` names a
// host-side stand-in, not device memory: its device address is looked up once
// per device (with that device current) and only that address is handed to
// kernels.  Every call on a GPU shares the array; it needs no clearing (the
// partition kernel writes every partial the merge reads).
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch` (looked up on its first use there).
i8kv_status scratch_of_current_device(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return I8KV_ERR_LAUNCH;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return I8KV_ERR_LAUNCH;
    }
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return I8KV_OK;
}

}  // namespace

extern "C" {

size_t i8kv_paged_decode_noalloc_max_bytes(void) { return kNoAllocScratchBytes; }

i8kv_status i8kv_paged_decode_int8_noalloc(const i8kv_cache_desc* desc, int32_t num_seqs,
                                           const int8_t* q_int8, const float* q_scale,
                                           const int8_t* k_cache, const int8_t* v_cache,
                                           const float* k_scale, const float* v_scale,
                                           const int32_t* block_tables,
                                           int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                           int32_t max_seq_len, int32_t partition_size,
                                           int32_t w_group, float softmax_scale, float* out,
                                           i8kv_stream_t stream) {
  // sizes first: a call that does not fit the fixed array is rejected before
  // the device is touched
  const i8kv_status sd = check_desc(desc);
  if (sd != I8KV_OK) return sd;
  if (num_seqs > 0 && max_seq_len >= 0 && max_seq_len <= kMaxSeqLen &&
      partition_size == kPartition) {
    const DecodePlan p = make_decode_plan(num_seqs, desc->num_kv_heads,
                                          desc->num_q_heads / desc->num_kv_heads,
                                          desc->head_dim, max_seq_len);
    if (p.bytes > kNoAllocScratchBytes) return I8KV_ERR_WORKSPACE;
  }
  void* ws = nullptr;
  const i8kv_status ss = scratch_of_current_device(&ws);
  if (ss != I8KV_OK) return ss;
  return run_decode(desc, num_seqs, q_int8, q_scale, k_cache, v_cache, k_scale, v_scale,
                    block_tables, max_blocks_per_seq, seq_lens, max_seq_len, partition_size,
                    w_group, softmax_scale, ws, kNoAllocScratchBytes, out, nullptr, stream);
}

size_t i8kv_prefix_prefill_workspace_bytes(const i8kv_cache_desc* desc, int32_t num_seqs,
                                           int32_t total_q) {
  (void)desc;
  (void)num_seqs;
  (void)total_q;
  return 0;
}

i8kv_status i8kv_prefix_prefill_int8(const i8kv_cache_desc* desc, int32_t num_seqs,
                                     int32_t total_q, int32_t max_query_len,
                                     const int8_t* q_int8, const float* q_scale,
                                     const int32_t* query_start_loc, const int32_t* seq_lens,
                                     const int8_t* k_cache, const int8_t* v_cache,
                                     const float* k_scale, const float* v_scale,
                                     const int32_t* block_tables, int32_t max_blocks_per_seq,
                                     int32_t w_group, float softmax_scale, void* workspace,
                                     size_t workspace_bytes, float* out,
                                     i8kv_stream_t stream) {
  return run_prefill(desc, num_seqs, total_q, max_query_len, q_int8, q_scale, query_start_loc,
                     seq_lens, k_cache, v_cache, k_scale, v_scale, block_tables,
                     max_blocks_per_seq, w_group, softmax_scale, workspace, workspace_bytes, out,
                     stream, false);
}

i8kv_status i8kv_prefix_prefill_uint8w(const i8kv_cache_desc* desc, int32_t num_seqs,
                                       int32_t total_q, int32_t max_query_len,
                                       const int8_t* q_int8, const float* q_scale,
                                       const int32_t* query_start_loc, const int32_t* seq_lens,
                                       const int8_t* k_cache, const int8_t* v_cache,
                                       const float* k_scale, const float* v_scale,
                                       const int32_t* block_tables, int32_t max_blocks_per_seq,
                                       int32_t w_group, float softmax_scale, void* workspace,
                                       size_t workspace_bytes, float* out,
                                       i8kv_stream_t stream) {
  return run_prefill(desc, num_seqs, total_q, max_query_len, q_int8, q_scale, query_start_loc,
                     seq_lens, k_cache, v_cache, k_scale, v_scale, block_tables,
                     max_blocks_per_seq, w_group, softmax_scale, workspace, workspace_bytes, out,
                     stream, false, nullptr, /*w_uint8=*/true);
}

i8kv_status i8kv_prefix_prefill_ex(const i8kv_cache_desc* desc, const i8kv_prefill_opts* opts,
                                   int32_t num_seqs, int32_t total_q, int32_t max_query_len,
                                   const int8_t* q_int8, const float* q_scale,
                                   const int32_t* query_start_loc, const int32_t* seq_lens,
                                   const int8_t* k_cache, const int8_t* v_cache,
                                   const float* k_scale, const float* v_scale,
                                   const int32_t* block_tables, int32_t max_blocks_per_seq,
                                   void* out, i8kv_stream_t stream) {
  if (!opts) return I8KV_ERR_NULL;
  if (opts->pv != I8KV_PV_INT8 && opts->pv != I8KV_PV_BF16 && opts->pv != I8KV_PV_UINT8)
    return I8KV_ERR_UNSUPPORTED;
  if (opts->out_bf16 != 0 && opts->out_bf16 != 1) return I8KV_ERR_INVALID_ARG;
  const bool bf16 = opts->pv == I8KV_PV_BF16;
  return run_prefill(desc, num_seqs, total_q, max_query_len, q_int8, q_scale, query_start_loc,
                     seq_lens, k_cache, v_cache, k_scale, v_scale, block_tables,
                     max_blocks_per_seq, bf16 ? 64 : opts->w_group, opts->softmax_scale, nullptr,
                     0, opts->out_bf16 ? nullptr : static_cast<float*>(out), stream, bf16,
                     nullptr, opts->pv == I8KV_PV_UINT8,
                     opts->out_bf16 ? static_cast<uint16_t*>(out) : nullptr);
}

i8kv_status i8kv_prefix_prefill_bf16pv(const i8kv_cache_desc* desc, int32_t num_seqs,
                                       int32_t total_q, int32_t max_query_len,
                                       const int8_t* q_int8, const float* q_scale,
                                       const int32_t* query_start_loc, const int32_t* seq_lens,
                                       const int8_t* k_cache, const int8_t* v_cache,
                                       const float* k_scale, const float* v_scale,
                                       const int32_t* block_tables, int32_t max_blocks_per_seq,
                                       float softmax_scale, void* workspace,
                                       size_t workspace_bytes, float* out,
                                       i8kv_stream_t stream) {
  return run_prefill(desc, num_seqs, total_q, max_query_len, q_int8, q_scale, query_start_loc,
                     seq_lens, k_cache, v_cache, k_scale, v_scale, block_tables,
                     max_blocks_per_seq, 64, softmax_scale, workspace, workspace_bytes, out,
                     stream, true);
}

i8kv_status i8kv_prefix_prefill_bf16qk(const i8kv_cache_desc* desc, int32_t num_seqs,
                                       int32_t total_q, int32_t max_query_len,
                                       const uint16_t* query_bf16,
                                       const int32_t* query_start_loc, const int32_t* seq_lens,
                                       const int8_t* k_cache, const int8_t* v_cache,
                                       const float* k_scale, const float* v_scale,
                                       const int32_t* block_tables, int32_t max_blocks_per_seq,
                                       int32_t w_group, float softmax_scale, void* workspace,
                                       size_t workspace_bytes, float* out,
                                       i8kv_stream_t stream) {
  if (!query_bf16) return I8KV_ERR_NULL;
  return run_prefill(desc, num_seqs, total_q, max_query_len, nullptr, nullptr, query_start_loc,
                     seq_lens, k_cache, v_cache, k_scale, v_scale, block_tables,
                     max_blocks_per_seq, w_group, softmax_scale, workspace, workspace_bytes, out,
                     stream, false, query_bf16);
}

}  // extern "C"
