"""Paged attention over an INT8 KV cache on AMD MI355X (gfx950).

Python binding of libi8kv.so.  Every step of the computation runs in the HIP
kernels behind the C ABI (include/i8kv.h); this package only marshals
arguments (torch tensors or raw device pointers) and checks shapes on the
host.  Importing it does not load the library; the first call does, and it
fails loudly if the library has not been built -- there is no fallback.

    kv_quantize_write(desc, key, value, slot_mapping, cache, query=None, ...)
    kv_quantize_write_rope(desc, key, value, slot_mapping, positions, cos_sin,
                           cache, query=None, ...)
    paged_decode_workspace_bytes(desc, num_seqs, max_seq_len)
    paged_decode_int8(desc, q_int8, q_scale, cache, block_tables, seq_lens, ...)
    paged_decode_partials(desc, q_int8, q_scale, cache, block_tables, seq_lens, ...)
    paged_decode_int8_noalloc(desc, q_int8, q_scale, cache, block_tables, seq_lens, ...)
    paged_decode_merge(desc, seq_lens, max_seq_len, workspace, ...)
    paged_decode_bf16pv(desc, q_int8, q_scale, cache, block_tables, seq_lens, ...)
    paged_decode_bf16qk(desc, query, cache, block_tables, seq_lens, ...)
    paged_decode_uint8w(desc, q_int8, q_scale, cache, block_tables, seq_lens, ...)
    paged_decode_ex(desc, q_int8, q_scale, cache, block_tables, seq_lens, max_seq_len,
                    queries_per_seq=1, pv="int8", w_group=32, out_bf16=False, ...)
    prefix_prefill_int8(desc, q_int8, q_scale, query_start_loc, seq_lens,
                        cache, block_tables, ...)
    prefix_prefill_bf16pv(desc, q_int8, q_scale, query_start_loc, seq_lens,
                          cache, block_tables, ...)
    prefix_prefill_bf16qk(desc, query, query_start_loc, seq_lens, cache, block_tables, ...)
    prefix_prefill_uint8w(desc, q_int8, q_scale, query_start_loc, seq_lens, cache, ...)
    prefix_prefill_ex(desc, q_int8, q_scale, query_start_loc, seq_lens, cache, block_tables,
                      max_query_len, pv="int8", w_group=32, out_bf16=False, ...)
    decode_step_int8(desc, key, value, query, cache, block_tables, seq_lens, ...)
"""
from ._binding import (  # noqa: F401
    CacheDesc,
    DecodeOpts,
    I8KVError,
    PagedCache,
    PrefillOpts,
    abi_version,
    decode_step_int8,
    kv_quantize_write,
    kv_quantize_write_rope,
    lib_path,
    load_library,
    paged_decode_bf16pv,
    paged_decode_bf16qk,
    paged_decode_ex,
    paged_decode_ex_workspace_bytes,
    paged_decode_int8,
    paged_decode_int8_noalloc,
    paged_decode_merge,
    paged_decode_noalloc_max_bytes,
    paged_decode_partials,
    paged_decode_uint8w,
    paged_decode_workspace_bytes,
    prefix_prefill_bf16pv,
    prefix_prefill_bf16qk,
    prefix_prefill_ex,
    prefix_prefill_int8,
    prefix_prefill_uint8w,
    prefix_prefill_workspace_bytes,
    status_string,
)
