// Fused KV producer: per-(token, head) symmetric int8 quantization of K, V
// (and optionally Q) with the paged cache write, in one kernel.
//
// Follows the page "INT8 KV and INT8 MMAC attention inference optimisation on
// a gfx936 DCU": section 2.1 (amax/127 scale, round, clamp to +-127, safe
// amax = 0), section 2.2 (read Q/K/V once, wave-level absmax, quantize, write
// the int8 pages and fp32 scales, no bf16 write-back, Q quantized once for
// reuse) and section 2.3 (K [blocks, Hkv, D/16, 16, 16], V [blocks, Hkv, D, 16],
// scales [blocks, 16, Hkv]).
//
// Mapping: a work item is one vector kind (a K head, a V head or a Q head) of
// TPW consecutive tokens, done by one wave; lane l owns the D/64 consecutive
// elements l*D/64 .. of each vector, so an absmax is one wave reduction and
// each lane's K bytes are contiguous inside one 16-byte head-dim chunk.
//  - Chunks (TPW = 16, one page's worth): all 16 loads are issued before any
//    arithmetic, the 16 wave maxima come out of one reduce-scatter, and when
//    the 16 tokens fill one page the lane holds whole 16-byte V rows (the
//    [D, 16] V page needs no transpose through LDS).
//  - Few tokens (TPW = 1): one wave per vector, for the shortest latency.
//
// With positions given, Q and K are first turned by the rotary embedding of
// their token's position (section 2.2 lists RoPE inside the producer): the
// rotate-half pairing, from a caller-given cos | sin table -- rope_wave_vector
// over the first rotary_dim < D dims, rope_wave_vector_full (table rows
// prefetched, pairs exchanged by v_permlane32_swap) over the whole head.
#include "device_common.hpp"
#include "kernels.hpp"

namespace i8kv {

constexpr int kProducerWaves = 4;      // waves per workgroup
constexpr int kChunkTokens = 16;       // TPW of the chunk kernel
constexpr int kChunkMinTokens = 128;   // fewer tokens: one vector per wave (lower latency)
// Rotation modes: none; over the first rotary_dim < D dims (table entries
// read where they are used); over the whole head (rows prefetched).
enum : int { kRopeNone = 0, kRopePartial = 1, kRopeFull = 2 };

// One work item: vector kind `kind` (0 K, 1 V, 2 Q) of head h for the tokens
// t0 .. t0 + nt - 1; src points at token t0's vector, stride is the distance
// (in elements) between consecutive tokens' vectors.
struct ProducerItem {
  const uint16_t* src;
  int64_t stride, t0;
  int kind, h, nt;
};

template <int D, int TPW>
__device__ __forceinline__ ProducerItem producer_item(const ProducerArgs& a, uint32_t item,
                                                      uint32_t per_tok) {
  ProducerItem it;
  it.t0 = (int64_t)(item / per_tok) * TPW;
  const int r = (int)(item % per_tok);
  it.nt = (int)min<int64_t>(TPW, a.num_tokens - it.t0);
  if (r < a.num_kv_heads) {
    it.kind = 0;
    it.h = r;
    it.src = a.key + (it.t0 * a.num_kv_heads + it.h) * D;
    it.stride = (int64_t)a.num_kv_heads * D;
  } else if (r < 2 * a.num_kv_heads) {
    it.kind = 1;
    it.h = r - a.num_kv_heads;
    it.src = a.value + (it.t0 * a.num_kv_heads + it.h) * D;
    it.stride = (int64_t)a.num_kv_heads * D;
  } else {
    it.kind = 2;
    it.h = r - 2 * a.num_kv_heads;
    it.src = a.query + (it.t0 * a.num_q_heads + it.h) * D;
    it.stride = (int64_t)a.num_q_heads * D;
  }
  return it;
}

// A position outside the table is clamped into it: the result is then
// meaningless, but no read leaves the table.
__device__ __forceinline__ int32_t clamped_pos(const ProducerArgs& a, int32_t p) {
  return min(max(p, 0), a.max_position - 1);
}

// What a wave loads for one item: the bf16 words, and in lane i token
// min(i, nt - 1)'s raw slot and position (checked where they are used).
template <int D, int TPW, int ROPE>
struct ProducerStage {
  uint2 raw[TPW];
  int32_t slot, pos;
  // Chunk items with rotation over the whole head (kRopeFull): token i's
  // table row, lane l holding its entries D/64 l .. (cosines in lanes 0-31,
  // sines in lanes 32-63).
  float cs[ROPE == kRopeFull && TPW > 1 ? TPW : 1][D / kWave];
};

// Issues every load of an item.  All loads are unconditional (a tail group
// re-reads its last token), so they stay in flight together and nothing
// waits for them until the item is finished.
template <int D, int TPW, int ROPE>
__device__ __forceinline__ void producer_load(const ProducerArgs& a, const ProducerItem& it,
                                              int lane, ProducerStage<D, TPW, ROPE>& st) {
  // slot and position first: waiting for them then leaves the bulk in flight
  const int64_t tl = it.t0 + min(lane, it.nt - 1);
  st.slot = a.slot_mapping[tl];
  if constexpr (ROPE) st.pos = a.positions[tl];
#pragma unroll
  for (int i = 0; i < TPW; ++i)
    st.raw[i] = load_wave_vector<D, true>(it.src + min(i, it.nt - 1) * it.stride, lane);
  if constexpr (ROPE == kRopeFull && TPW > 1) {
    // The table rows of all the item's tokens, issued before any of them is
    // used (one coalesced row per token), so that their latency overlaps
    // the bulk loads' instead of following it token by token.
    if (it.kind != 1) {
      constexpr int EPL = D / kWave;
#pragma unroll
      for (int i = 0; i < TPW; ++i) {
        const int pos = clamped_pos(a, __builtin_amdgcn_readlane(st.pos, i));
        const float* row = a.cos_sin + (int64_t)pos * D + EPL * lane;
#pragma unroll
        for (int e = 0; e < EPL; ++e) st.cs[i][e] = row[e];
      }
    }
  }
}

// Lane i's cache slot for token i, or -1 for no write: lanes past the item,
// Q items, negative slots and slots past the cache.
__device__ __forceinline__ int32_t checked_slot(const ProducerArgs& a, const ProducerItem& it,
                                                int lane, int32_t s) {
  const bool ok = it.kind < 2 && lane < it.nt && s >= 0 &&
                  (int64_t)s < (int64_t)a.num_blocks * kBlockSize;
  return ok ? s : -1;
}

// Page-aligned V write: the 16 tokens of this wave fill offsets 0..15 of one
// page in order, so lane l holds all 16 bytes of its D/64 head-dim rows
// (row d = l*D/64 + j gets byte i from token i's j-th code).  The rows pass
// through LDS (row r at (r + r/16) * 16 bytes: conflict-free both ways) so
// that the page ([D][16 tokens], 16 D bytes) goes out as D/64 contiguous 1 KB
// store instructions.
template <int D>
__device__ __forceinline__ void store_v_page_staged(int8_t* page, int lane,
                                                    const uint32_t (&codes)[kChunkTokens],
                                                    uint8_t* lds) {
  constexpr int EPL = D / kWave;
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      w[k] = 0;
#pragma unroll
      for (int m = 0; m < 4; ++m) w[k] |= ((codes[4 * k + m] >> (8 * j)) & 0xffu) << (8 * m);
    }
    const int r = lane * EPL + j;
    *reinterpret_cast<uint4*>(lds + (r + r / 16) * 16) = make_uint4(w[0], w[1], w[2], w[3]);
  }
  asm volatile("" ::: "memory");  // a wave's LDS accesses complete in order
  // Pages (and Q rows below) are written once and not read back by this
  // call: non-temporal stores (2242-token chunk 17.6 -> 15.9 us, with RoPE
  // 21.5 -> 18.3 us, against ordinary stores).
#pragma unroll
  for (int i = 0; i < D / 64; ++i) {
    const int r = 64 * i + lane;
    __builtin_nontemporal_store(*reinterpret_cast<const v4u*>(lds + (r + r / 16) * 16),
                                reinterpret_cast<v4u*>(page + r * 16));
  }
}

// Per-wave LDS staging of the chunk kernel: a K page with its D/16 chunks
// padded to 272 bytes (conflict-free for the per-token writes); the same
// bytes hold the padded V page image or the 16 x D bytes of Q rows.
template <int D>
constexpr int kStageBytes = (D / 16) * (kChunkTokens * 16 + 16);

template <int D>
__device__ __forceinline__ void lds_put_codes(uint8_t* p, uint32_t codes) {
  constexpr int EPL = D / kWave;
  if constexpr (EPL == 4) *reinterpret_cast<uint32_t*>(p) = codes;
  else if constexpr (EPL == 2) *reinterpret_cast<uint16_t*>(p) = (uint16_t)codes;
  else *p = (uint8_t)codes;
}

// Q codes of the wave's tokens through LDS: written as [token][D] rows, read
// back 16 bytes per lane so that every store instruction covers 1 KB of
// whole rows (1024 / D tokens) instead of 4 bytes per lane of one token.
template <int D>
__device__ __forceinline__ void store_q_staged(int8_t* q0, int64_t token_stride, int nt, int lane,
                                               const uint32_t (&codes)[kChunkTokens],
                                               uint8_t* lds) {
  constexpr int EPL = D / kWave;
#pragma unroll
  for (int t = 0; t < kChunkTokens; ++t) lds_put_codes<D>(lds + t * D + lane * EPL, codes[t]);
  asm volatile("" ::: "memory");  // a wave's LDS accesses complete in order
#pragma unroll
  for (int j = 0; j < D / 64; ++j) {
    const int off = j * 1024 + lane * 16;
    const int t = off / D;
    const uint4 v = *reinterpret_cast<const uint4*>(lds + off);
    if (t < nt)
      __builtin_nontemporal_store(v4u{v.x, v.y, v.z, v.w},
                                  reinterpret_cast<v4u*>(q0 + t * token_stride + off % D));
  }
}

// A whole K page ([D/16][16 tokens][16 bytes], 16 D bytes) through LDS: each
// lane's per-token bytes land in the padded page image, and the page goes
// out as D/64 contiguous 1 KB store instructions.
template <int D>
__device__ __forceinline__ void store_k_page_staged(int8_t* page, int lane,
                                                    const uint32_t (&codes)[kChunkTokens],
                                                    uint8_t* lds) {
  constexpr int EPL = D / kWave;
  constexpr int CS = kChunkTokens * 16 + 16;  // padded chunk stride
  uint8_t* w = lds + (lane * EPL / 16) * CS + (lane * EPL) % 16;
#pragma unroll
  for (int t = 0; t < kChunkTokens; ++t) lds_put_codes<D>(w + t * 16, codes[t]);
  asm volatile("" ::: "memory");
#pragma unroll
  for (int j = 0; j < D / 64; ++j) {
    const int r = 64 * j + lane;  // row (chunk r / 16, token r % 16)
    const uint4 v = *reinterpret_cast<const uint4*>(lds + (r / 16) * CS + (r % 16) * 16);
    __builtin_nontemporal_store(v4u{v.x, v.y, v.z, v.w}, reinterpret_cast<v4u*>(page + r * 16));
  }
}

// Quantizes and stores one loaded item.  Lane i < nt ends up with token i's
// scale, so the scales go out in one store.
template <int D, int TPW, int ROPE>
__device__ __forceinline__ void producer_finish(const ProducerArgs& a, const ProducerItem& it,
                                                int lane, const ProducerStage<D, TPW, ROPE>& st,
                                                uint8_t* lds) {
  constexpr int EPL = D / kWave;
  uint32_t codes[TPW];
  float my_scale = 0.0f;
  if constexpr (TPW == 1) {
    float x[EPL];
    unpack_wave_vector<D>(st.raw[0], x);
    if constexpr (ROPE) {
      if (it.kind != 1) {  // V is not rotated
        const int pos = clamped_pos(a, __builtin_amdgcn_readfirstlane(st.pos));
        rope_wave_vector<D>(x, lane, a.cos_sin + (int64_t)pos * a.rotary_dim, a.rotary_dim);
      }
    }
    codes[0] = quantize_wave_values<D>(x, my_scale);
  } else {
    // Straight-line over all 16 (a tail group's extra tokens are recomputed
    // copies of its last one and never stored).  First each lane's partial
    // maxima, then all 16 wave maxima in one reduce-scatter (lane 4i ends
    // with token i's), the scales with one division per lane, and the codes
    // from each token's scale read back as a wave constant.  Without rotation
    // the bf16 words are unpacked again for the codes rather than kept as
    // fp32 values.
    float xr[ROPE ? TPW : 1][EPL];
    float pm[TPW];
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      float x[EPL];
      unpack_wave_vector<D>(st.raw[i], x);
      if constexpr (ROPE) {
        if (it.kind != 1) {
          if constexpr (ROPE == kRopeFull) {
            rope_wave_vector_full<D>(x, lane, st.cs[i]);
          } else {
            const int pos = clamped_pos(a, __builtin_amdgcn_readlane(st.pos, i));
            rope_wave_vector<D>(x, lane, a.cos_sin + (int64_t)pos * a.rotary_dim, a.rotary_dim);
          }
        }
#pragma unroll
        for (int e = 0; e < EPL; ++e) xr[i][e] = x[e];
      }
      pm[i] = 0.0f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) pm[i] = fmaxf(pm[i], fabsf(x[e]));
    }
    const float amax = wave_max_scatter16(pm, lane);
    const float s = amax / 127.0f;
    const float sd = amax != 0.0f ? s : 1.0f;
    const float rs = 1.0f / sd;
    my_scale = __shfl(s, 4 * lane, kWave);  // token `lane`'s, for lane < 16
    const uint64_t subnormal = __ballot(!(sd >= 0x1p-126f));  // bit 4i: token i's scale
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const float sd_i = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sd), 4 * i));
      const float rs_i = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(rs), 4 * i));
      const bool div_i = (subnormal >> (4 * i)) & 1;
      if constexpr (ROPE) {
        codes[i] = quantize_codes_rs<EPL>(xr[i], sd_i, rs_i, div_i);
      } else {
        float x[EPL];
        unpack_wave_vector<D>(st.raw[i], x);
        codes[i] = quantize_codes_rs<EPL>(x, sd_i, rs_i, div_i);
      }
    }
  }

  const int d0 = lane * EPL;
  if (it.kind == 2) {
    int8_t* q0 = a.q_int8 + (it.t0 * a.num_q_heads + it.h) * D;
    if constexpr (TPW == kChunkTokens) {
      store_q_staged<D>(q0, (int64_t)a.num_q_heads * D, it.nt, lane, codes, lds);
      if (lane < it.nt) a.q_scale[(it.t0 + lane) * a.num_q_heads + it.h] = my_scale;
      return;
    }
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      if (i < it.nt) {
        int8_t* dst = a.q_int8 + ((it.t0 + i) * a.num_q_heads + it.h) * D + d0;
        if constexpr (EPL == 4) *reinterpret_cast<uint32_t*>(dst) = codes[i];
        else if constexpr (EPL == 2) *reinterpret_cast<uint16_t*>(dst) = (uint16_t)codes[i];
        else *dst = (int8_t)codes[i];
      }
    }
    if (lane < it.nt) a.q_scale[(it.t0 + lane) * a.num_q_heads + it.h] = my_scale;
    return;
  }

  const int Hkv = a.num_kv_heads;
  const int32_t my_slot = checked_slot(a, it, lane, st.slot);
  bool paged = false;
  if constexpr (TPW == kChunkTokens) {
    const int32_t base = __builtin_amdgcn_readfirstlane(my_slot);
    const bool off_run = lane < TPW && my_slot != base + lane;
    paged = it.nt == TPW && base >= 0 && base % kBlockSize == 0 && __ballot(off_run) == 0;
    if (paged) {
      const int64_t blk = base / kBlockSize;
      if (it.kind == 1)
        store_v_page_staged<D>(a.v_cache + (blk * Hkv + it.h) * D * kBlockSize, lane, codes, lds);
      else
        store_k_page_staged<D>(a.k_cache + (blk * Hkv + it.h) * D * kBlockSize, lane, codes, lds);
    }
  }
  if (!paged) {
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int32_t slot = __builtin_amdgcn_readlane(my_slot, i);
      if (i < it.nt && slot >= 0) {
        if (it.kind == 0)
          store_k_token<D>(a.k_cache, slot / kBlockSize, it.h, Hkv, slot % kBlockSize, lane, codes[i]);
        else
          store_v_token<D>(a.v_cache, slot / kBlockSize, it.h, Hkv, slot % kBlockSize, lane, codes[i]);
      }
    }
  }
  if (my_slot >= 0) {
    const int64_t sidx = (int64_t)my_slot * Hkv + it.h;  // [blocks, 16, Hkv]
    (it.kind == 0 ? a.k_scale : a.v_scale)[sidx] = my_scale;
  }
}

// Workgroups are handed to the 8 XCDs in turn (workgroup b to XCD b % 8),
// and each XCD has its own L2.  Numbering the work so that XCD x gets the
// x-th contiguous eighth of it keeps the items of one token chunk (which
// read the same rotary-table rows) on one XCD, so each row comes from HBM
// once instead of once per XCD.  A bijection of 0 .. n - 1 whatever the
// actual placement: only locality depends on it.
constexpr uint32_t kXcds = 8;
__device__ __forceinline__ uint32_t xcd_block(uint32_t b, uint32_t n) {
  const uint32_t x = b % kXcds, slot = b / kXcds, q = n / kXcds, r = n % kXcds;
  return x * q + min(x, r) + slot;
}

template <int D, int TPW, int ROPE>
__global__ __launch_bounds__(kProducerWaves * kWave) void kv_quantize_write_kernel(ProducerArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const uint32_t wid = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  // Item counts fit in 32 bits (checked at launch).
  const uint32_t per_tok = 2 * a.num_kv_heads + (a.query ? a.num_q_heads : 0);
  const uint32_t n_items = ((uint32_t)a.num_tokens + TPW - 1) / TPW * per_tok;
  // The rotating kernels number their work XCD by XCD (4096-token chunk with
  // rotation: 33.4 -> 28.3 us together with the prefetched table rows); the
  // others keep the plain order (the remap measured +0.6 us at 4096 tokens
  // and -0.8 us at 2242 there).
  const uint32_t blk = ROPE ? xcd_block(blockIdx.x, gridDim.x) : blockIdx.x;
  const uint32_t item = blk * kProducerWaves + wid;
  if (item >= n_items) return;  // wave-uniform
  const ProducerItem it = producer_item<D, TPW>(a, item, per_tok);
  ProducerStage<D, TPW, ROPE> st;
  producer_load<D, TPW, ROPE>(a, it, lane, st);
  if constexpr (TPW == kChunkTokens) {
    __shared__ uint4 stage[kProducerWaves][kStageBytes<D> / 16];
    producer_finish<D, TPW, ROPE>(a, it, lane, st, reinterpret_cast<uint8_t*>(stage[wid]));
  } else {
    producer_finish<D, TPW, ROPE>(a, it, lane, st, nullptr);
  }
}

template <int D, int ROPE>
hipError_t launch_producer(const ProducerArgs& a, hipStream_t stream) {
  const int64_t per_tok = 2 * (int64_t)a.num_kv_heads + (a.query ? a.num_q_heads : 0);
  const int tpw = a.num_tokens < kChunkMinTokens ? 1 : kChunkTokens;
  const int64_t items = ((int64_t)a.num_tokens + tpw - 1) / tpw * per_tok;
  if (items > 0x7fff0000) return hipErrorInvalidValue;  // 32-bit item counters
  const int64_t want = (items + kProducerWaves - 1) / kProducerWaves;
  dim3 block(kProducerWaves * kWave);
  if (tpw == 1)
    hipLaunchKernelGGL((kv_quantize_write_kernel<D, 1, ROPE>), dim3((unsigned)want), block, 0,
                       stream, a);
  else
    hipLaunchKernelGGL((kv_quantize_write_kernel<D, kChunkTokens, ROPE>), dim3((unsigned)want),
                       block, 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_kv_quantize_write(const ProducerArgs& a, hipStream_t stream) {
  if (a.num_tokens <= 0) return hipSuccess;
  const int mode = a.positions == nullptr ? kRopeNone
                   : a.rotary_dim == a.head_dim ? kRopeFull : kRopePartial;
  switch (a.head_dim * 4 + mode) {
    case 64 * 4 + kRopeNone: return launch_producer<64, kRopeNone>(a, stream);
    case 64 * 4 + kRopePartial: return launch_producer<64, kRopePartial>(a, stream);
    case 64 * 4 + kRopeFull: return launch_producer<64, kRopeFull>(a, stream);
    case 128 * 4 + kRopeNone: return launch_producer<128, kRopeNone>(a, stream);
    case 128 * 4 + kRopePartial: return launch_producer<128, kRopePartial>(a, stream);
    case 128 * 4 + kRopeFull: return launch_producer<128, kRopeFull>(a, stream);
    case 256 * 4 + kRopeNone: return launch_producer<256, kRopeNone>(a, stream);
    case 256 * 4 + kRopePartial: return launch_producer<256, kRopePartial>(a, stream);
    case 256 * 4 + kRopeFull: return launch_producer<256, kRopeFull>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace i8kv
