// Device helpers shared by the i8kv HIP kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.hpp"

namespace i8kv {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_bits_to_float(uint32_t b) {
  return __uint_as_float(b << 16);
}

// Quantization rule of the producer: q = clamp(round(x / s), -127, 127) with
// IEEE division and rounding half away from zero (roundf).
__device__ __forceinline__ int quantize_code(float x, float s) {
  float r = roundf(x / s);
  r = fminf(fmaxf(r, -127.0f), 127.0f);
  return (int)r;
}

// Butterfly reductions inside aligned groups of `width` lanes (width <= 64).
template <int width>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
  for (int o = width / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

template <int width>
__device__ __forceinline__ double group_sum(double v) {
#pragma unroll
  for (int o = width / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

template <int width>
__device__ __forceinline__ float group_sumf(float v) {
#pragma unroll
  for (int o = width / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Correctly rounded fp32 exponential: e^x evaluated in fp64 and rounded once.
__device__ __forceinline__ float exp_f32_rn(float x) {
  return (float)exp((double)x);
}

}  // namespace i8kv
