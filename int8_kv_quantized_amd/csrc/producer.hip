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

  float x[EPL];
  if constexpr (EPL == 4) {
    const uint2 raw = *reinterpret_cast<const uint2*>(src + lane * 4);
    x[0] = bf16_bits_to_float(raw.x & 0xffffu);
    x[1] = bf16_bits_to_float(raw.x >> 16);
    x[2] = bf16_bits_to_float(raw.y & 0xffffu);
    x[3] = bf16_bits_to_float(raw.y >> 16);
  } else if constexpr (EPL == 2) {
    const uint32_t raw = *reinterpret_cast<const uint32_t*>(src + lane * 2);
    x[0] = bf16_bits_to_float(raw & 0xffffu);
    x[1] = bf16_bits_to_float(raw >> 16);
  } else {
    x[0] = bf16_bits_to_float(src[lane]);
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < EPL; ++i) amax = fmaxf(amax, fabsf(x[i]));
  amax = group_max<kWave>(amax);

  float s = 0.0f;
  uint32_t packed = 0;
  if (amax != 0.0f) {
    s = amax / 127.0f;
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      packed |= ((uint32_t)(quantize_code(x[i], s) & 0xff)) << (8 * i);
  }

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
    // K [blk, h, d/16, off, d%16]: this lane's EPL bytes sit in one chunk.
    int8_t* dst = a.k_cache +
                  (((blk * a.num_kv_heads + h) * (D / 16) + d0 / 16) * kBlockSize + off) * 16 +
                  d0 % 16;
    if constexpr (EPL == 4) *reinterpret_cast<uint32_t*>(dst) = packed;
    else if constexpr (EPL == 2) *reinterpret_cast<uint16_t*>(dst) = (uint16_t)packed;
    else *dst = (int8_t)packed;
    if (lane == 0) a.k_scale[sidx] = s;
  } else {
    // V [blk, h, d, off]: tokens innermost, one byte per (d, off).
    int8_t* dst = a.v_cache + ((blk * a.num_kv_heads + h) * D + d0) * kBlockSize + off;
#pragma unroll
    for (int i = 0; i < EPL; ++i) dst[i * kBlockSize] = (int8_t)(packed >> (8 * i));
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
