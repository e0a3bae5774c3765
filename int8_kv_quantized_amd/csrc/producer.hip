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
// Mapping: one wave per vector of D elements; lane l owns the D/64
// consecutive elements l*D/64 .. so the absmax is one wave reduction and each
// lane's K bytes are contiguous inside one 16-byte head-dim chunk.
#include "device_common.hpp"
#include "kernels.hpp"

namespace i8kv {

template <int D>
__global__ __launch_bounds__(256) void kv_quantize_write_kernel(ProducerArgs a) {
  constexpr int EPL = D / kWave;  // 1, 2 or 4 elements per lane
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t vec = (int64_t)blockIdx.x * (blockDim.x / kWave) + (threadIdx.x / kWave);
  const int per_tok = 2 * a.num_kv_heads + (a.query ? a.num_q_heads : 0);
  if (vec >= (int64_t)a.num_tokens * per_tok) return;  // wave-uniform
  const int t = (int)(vec / per_tok);
  const int r = (int)(vec % per_tok);

  const uint16_t* src;
  int kind, h;
  if (r < a.num_kv_heads) {
    kind = 0;
    h = r;
    src = a.key + ((int64_t)t * a.num_kv_heads + h) * D;
  } else if (r < 2 * a.num_kv_heads) {
    kind = 1;
    h = r - a.num_kv_heads;
    src = a.value + ((int64_t)t * a.num_kv_heads + h) * D;
  } else {
    kind = 2;
    h = r - 2 * a.num_kv_heads;
    src = a.query + ((int64_t)t * a.num_q_heads + h) * D;
  }
  int32_t slot = 0;
  if (kind < 2) {
    slot = a.slot_mapping[t];
    // Negative slots skip the write; out-of-range slots are dropped too.
    if (slot < 0 || (int64_t)slot >= (int64_t)a.num_blocks * kBlockSize) return;
  }

  float s = 0.0f;
  const uint32_t packed = quantize_wave_vector<D>(load_wave_vector<D>(src, lane), s);

  const int d0 = lane * EPL;
  if (kind == 2) {
    int8_t* dst = a.q_int8 + ((int64_t)t * a.num_q_heads + h) * D + d0;
    if constexpr (EPL == 4) *reinterpret_cast<uint32_t*>(dst) = packed;
    else if constexpr (EPL == 2) *reinterpret_cast<uint16_t*>(dst) = (uint16_t)packed;
    else *dst = (int8_t)packed;
    if (lane == 0) a.q_scale[(int64_t)t * a.num_q_heads + h] = s;
    return;
  }
  const int64_t blk = slot / kBlockSize;
  const int off = slot % kBlockSize;
  const int64_t sidx = (blk * kBlockSize + off) * a.num_kv_heads + h;
  if (kind == 0) {
    store_k_token<D>(a.k_cache, blk, h, a.num_kv_heads, off, lane, packed);
    if (lane == 0) a.k_scale[sidx] = s;
  } else {
    store_v_token<D>(a.v_cache, blk, h, a.num_kv_heads, off, lane, packed);
    if (lane == 0) a.v_scale[sidx] = s;
  }
}

hipError_t launch_kv_quantize_write(const ProducerArgs& a, hipStream_t stream) {
  const int per_tok = 2 * a.num_kv_heads + (a.query ? a.num_q_heads : 0);
  const int64_t vecs = (int64_t)a.num_tokens * per_tok;
  if (vecs == 0) return hipSuccess;
  constexpr int kWavesPerBlock = 4;
  const int64_t blocks = (vecs + kWavesPerBlock - 1) / kWavesPerBlock;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  dim3 grid((unsigned)blocks), block(kWavesPerBlock * kWave);
  switch (a.head_dim) {
    case 64: hipLaunchKernelGGL(kv_quantize_write_kernel<64>, grid, block, 0, stream, a); break;
    case 128: hipLaunchKernelGGL(kv_quantize_write_kernel<128>, grid, block, 0, stream, a); break;
    case 256: hipLaunchKernelGGL(kv_quantize_write_kernel<256>, grid, block, 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace i8kv
