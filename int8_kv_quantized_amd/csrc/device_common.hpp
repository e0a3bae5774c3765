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

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

// Eight int8 values (bytes of lo, then hi) as bf16: exact, since |v| <= 128
// needs at most 8 significant bits; the bf16 bits are the top half of the
// fp32 value.
__device__ __forceinline__ v8bf i8x8_to_bf16(uint32_t lo, uint32_t hi) {
  uint32_t f[8];
#pragma unroll
  for (int k = 0; k < 8; ++k)
    f[k] = __float_as_uint((float)(int8_t)(((k < 4 ? lo : hi) >> (8 * (k & 3))) & 0xffu));
  v4u w;
#pragma unroll
  for (int k = 0; k < 4; ++k) w[k] = (f[2 * k] >> 16) | (f[2 * k + 1] & 0xffff0000u);
  return __builtin_bit_cast(v8bf, w);
}

// fp32 -> bf16 bits, round to nearest, ties to even (finite inputs).
__device__ __forceinline__ uint32_t bf16_rne_bits(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// Code of an already divided value: clamp(round(q), -127, 127).
__device__ __forceinline__ int round_code(float q) {
  return (int)fminf(fmaxf(roundf(q), -127.0f), 127.0f);
}

// The IEEE fp32 quotient a / b, given rb ~ 1/b in fp64 (relative error below
// 2^-51).  When a / b is a normal fp32 number it is never a rounding midpoint
// and lies at least ~2^-49 (relative) away from one, while a * rb carries a
// relative error below 2^-50.5, so rounding a * rb to fp32 gives the correctly
// rounded quotient.  A quotient in the fp32 subnormal range can be an exact
// midpoint of the coarser subnormal grid, so there the IEEE division is done.
__device__ __forceinline__ float div_f32_rn(float a, float b, double rb) {
  const double q = (double)a * rb;
  if (__builtin_fabs(q) < 0x1p-126) return a / b;
  return (float)q;
}

// 1/x for a positive, finite, normal fp64 x: the hardware estimate refined by
// two Newton steps, r' = r + r (1 - x r).  The result is within ~1 ulp of 1/x,
// well inside the 2^-51 that div_f32_rn needs; x = 0 gives a non-finite value.
__device__ __forceinline__ double rcp_f64(double x) {
  double r = __builtin_amdgcn_rcp(x);
  double e = __builtin_fma(-x, r, 1.0);
  r = __builtin_fma(r, e, r);
  e = __builtin_fma(-x, r, 1.0);
  return __builtin_fma(r, e, r);
}

// ---- cross-lane reductions inside aligned groups of `width` lanes ----------
// Within a 16-lane row: DPP quad_perm [1,0,3,2] and [2,3,0,1] (pairs at
// distance 1 and 2), row_half_mirror (lane i <-> 7-i of each 8) and
// row_mirror (i <-> 15-i): after each step every lane holds the reduction of
// its block, and the mirrors pair the two halves of the next larger block.
// Across rows: v_permlane16_swap / v_permlane32_swap return, for every lane,
// its own value and its partner's (rows 2k <-> 2k+1, halves), so op(r0, r1)
// completes the next level whichever of the two is the partner.
enum : int { kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140 };

template <int ctrl>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, ctrl, 0xF, 0xF, false);
}

struct MaxOp {
  __device__ float operator()(float a, float b) const { return fmaxf(a, b); }
};
struct AddOp {
  __device__ float operator()(float a, float b) const { return a + b; }
  __device__ double operator()(double a, double b) const { return a + b; }
};

__device__ __forceinline__ float bits_f(uint32_t u) { return __uint_as_float(u); }
__device__ __forceinline__ uint32_t f_bits(float f) { return __float_as_uint(f); }

template <int ctrl>
__device__ __forceinline__ float dpp_f(float v) {
  return bits_f(dpp_u32<ctrl>(f_bits(v)));
}
template <int ctrl>
__device__ __forceinline__ double dpp_d(double v) {
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = dpp_u32<ctrl>((uint32_t)u), hi = dpp_u32<ctrl>((uint32_t)(u >> 32));
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

__device__ __forceinline__ void swap16(uint32_t v, uint32_t& a, uint32_t& b) {
  const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  a = r[0];
  b = r[1];
}
__device__ __forceinline__ void swap32(uint32_t v, uint32_t& a, uint32_t& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  a = r[0];
  b = r[1];
}

template <int width, typename Op>
__device__ __forceinline__ float group_reduce(float v, Op op) {
  if constexpr (width >= 2) v = op(v, dpp_f<kDppXor1>(v));
  if constexpr (width >= 4) v = op(v, dpp_f<kDppXor2>(v));
  if constexpr (width >= 8) v = op(v, dpp_f<kDppHalfMirror>(v));
  if constexpr (width >= 16) v = op(v, dpp_f<kDppMirror>(v));
  if constexpr (width >= 32) {
    uint32_t a, b;
    swap16(f_bits(v), a, b);
    v = op(bits_f(a), bits_f(b));
  }
  if constexpr (width >= 64) {
    uint32_t a, b;
    swap32(f_bits(v), a, b);
    v = op(bits_f(a), bits_f(b));
  }
  return v;
}

template <int width>
__device__ __forceinline__ double group_reduce_sum(double v) {
  if constexpr (width >= 2) v += dpp_d<kDppXor1>(v);
  if constexpr (width >= 4) v += dpp_d<kDppXor2>(v);
  if constexpr (width >= 8) v += dpp_d<kDppHalfMirror>(v);
  if constexpr (width >= 16) v += dpp_d<kDppMirror>(v);
  if constexpr (width >= 32) {
    const uint64_t u = (uint64_t)__double_as_longlong(v);
    uint32_t la, lb, ha, hb;
    swap16((uint32_t)u, la, lb);
    swap16((uint32_t)(u >> 32), ha, hb);
    v = __longlong_as_double((long long)(((uint64_t)ha << 32) | la)) +
        __longlong_as_double((long long)(((uint64_t)hb << 32) | lb));
  }
  if constexpr (width >= 64) {
    const uint64_t u = (uint64_t)__double_as_longlong(v);
    uint32_t la, lb, ha, hb;
    swap32((uint32_t)u, la, lb);
    swap32((uint32_t)(u >> 32), ha, hb);
    v = __longlong_as_double((long long)(((uint64_t)ha << 32) | la)) +
        __longlong_as_double((long long)(((uint64_t)hb << 32) | lb));
  }
  return v;
}

template <int width>
__device__ __forceinline__ float group_max(float v) {
  return group_reduce<width>(v, MaxOp{});
}
template <int width>
__device__ __forceinline__ float group_sumf(float v) {
  return group_reduce<width>(v, AddOp{});
}
template <int width>
__device__ __forceinline__ double group_sum(double v) {
  return group_reduce_sum<width>(v);
}

// fp32 exponential rounded once from an fp64 evaluation of e^x (relative
// error about 2^-42 before the final rounding, so the fp32 result is the
// correctly rounded one except within ~2^-18 of a rounding midpoint).
// Method: e^x = 2^t with t = x log2(e); t = n + f, n = rint(t), |f| <= 1/2;
// 2^f = e^(f ln 2) by its Taylor series to degree 10 (Horner); scale by 2^n.
__device__ __forceinline__ float exp_f32_rn(float x) {
  const double t = (double)x * 1.4426950408889634074;
  const double n = __builtin_rint(t);
  const double g = (t - n) * 0.69314718055994530942;
  double p = 2.7557319223985893e-07;          // 1/10!
  p = __builtin_fma(p, g, 2.7557319223985888e-06);  // 1/9!
  p = __builtin_fma(p, g, 2.4801587301587302e-05);  // 1/8!
  p = __builtin_fma(p, g, 1.9841269841269841e-04);  // 1/7!
  p = __builtin_fma(p, g, 1.3888888888888889e-03);  // 1/6!
  p = __builtin_fma(p, g, 8.3333333333333333e-03);  // 1/5!
  p = __builtin_fma(p, g, 4.1666666666666667e-02);  // 1/4!
  p = __builtin_fma(p, g, 1.6666666666666667e-01);  // 1/3!
  p = __builtin_fma(p, g, 0.5);
  p = __builtin_fma(p, g, 1.0);
  p = __builtin_fma(p, g, 1.0);
  return (float)__builtin_ldexp(p, (int)n);
}

// ---- one wave quantizes one D-vector of bf16 (the producer's rule) ---------
// Lane l owns the D/64 consecutive elements l*D/64 ..; `raw` holds their bf16
// bits (element i in bits 16i..16i+15).
template <int D>
__device__ __forceinline__ void unpack_wave_vector(uint2 raw, float (&x)[D / kWave]) {
#pragma unroll
  for (int i = 0; i < D / kWave; ++i) {
    const uint32_t word = i < 2 ? raw.x : raw.y;
    x[i] = bf16_bits_to_float((word >> (16 * (i & 1))) & 0xffffu);
  }
}

// Codes of a lane's n elements given the vector's scale s (amax / 127) as
//   sd = s, or 1 when amax = 0 (all elements are then zero), and rs = 1 / sd.
// Fast rule: qh = fma(x, rs, 128.5 + 2^-14) lies within 1.9e-5 of the IEEE
// quotient y = x / sd plus the same constant (|x| <= 127 sd, sd normal).  If
// fract(qh) >= 2^-13, y + 128 is more than 1e-4 from every half-integer and
// floor(qh) - 128 is the code clamp(round(y)) with ties away from zero (never
// a tie, never outside [-127, 127]); the biased code (1..255) is converted
// from the exact integer floor(qh) and the bias removed by flipping each
// byte's top bit.  A lane with an element too close to a half-integer, or a
// call with `divide` set (subnormal sd: 1 / sd may overflow), divides
// instead.  (Checked on the CPU exhaustively for every bf16 x and amax with a
// normal scale, and on random and near-midpoint fp32 inputs.)
template <int n>
__device__ __forceinline__ uint32_t quantize_codes_rs(const float (&x)[n], float sd, float rs,
                                                      bool divide) {
  static_assert(n >= 1 && n <= 4, "at most four codes per lane");
  constexpr uint32_t kFlip = n == 4 ? 0x80808080u : n == 2 ? 0x8080u : 0x80u;
  constexpr float kBias = 128.5f + 0x1p-14f;  // exact in fp32
  float qh[n];
  float fmin = 1.0f;
#pragma unroll
  for (int i = 0; i < n; ++i) {
    qh[i] = fmaf(x[i], rs, kBias);
    fmin = fminf(fmin, __builtin_amdgcn_fractf(qh[i]));
  }
  uint32_t packed = 0;
#pragma unroll
  for (int i = 0; i < n; ++i) packed = __builtin_amdgcn_cvt_pk_u8_f32(floorf(qh[i]), i, packed);
  packed ^= kFlip;
  if (divide || fmin < 0x1p-13f) {
    packed = 0;
#pragma unroll
    for (int i = 0; i < n; ++i) packed |= ((uint32_t)(quantize_code(x[i], sd) & 0xff)) << (8 * i);
  }
  return packed;
}

// Returns the lane's codes packed one byte per element and sets `scale`:
// amax = max |x| over the wave, scale = amax / 127 (IEEE), code =
// clamp(round(x / scale), -127, 127), and scale 0 with all-zero codes when
// amax = 0.
template <int D>
__device__ __forceinline__ uint32_t quantize_wave_values(const float (&x)[D / kWave], float& scale) {
  constexpr int EPL = D / kWave;
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < EPL; ++i) amax = fmaxf(amax, fabsf(x[i]));
  amax = group_max<kWave>(amax);
  const float s = amax / 127.0f;
  const float sd = amax != 0.0f ? s : 1.0f;
  scale = s;
  return quantize_codes_rs<EPL>(x, sd, 1.0f / sd, !(sd >= 0x1p-126f));
}

// Wave maxima of 16 per-lane non-negative floats at once (a reduce-scatter,
// on their bit patterns, whose unsigned order is the numeric order):
// afterwards lane l holds the maximum over all 64 lanes of value l >> 2.
// Each stage halves the values a lane keeps: v_permlane32_swap pairs the
// wave's halves (lanes 0-31 keep values 0-7, lanes 32-63 values 8-15),
// v_permlane16_swap pairs rows 2k and 2k+1, row_mirror pairs lane i with
// 15 - i and row_half_mirror i with 7 - i; two quad steps finish.
__device__ __forceinline__ float wave_max_scatter16(const float (&vf)[16], int lane) {
  uint32_t v[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) v[j] = f_bits(vf[j]);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const auto r = __builtin_amdgcn_permlane32_swap(v[j], v[j + 8], false, false);
    v[j] = max((uint32_t)r[0], (uint32_t)r[1]);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const auto r = __builtin_amdgcn_permlane16_swap(v[j], v[j + 4], false, false);
    v[j] = max((uint32_t)r[0], (uint32_t)r[1]);
  }
  const bool b3 = lane & 8;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const uint32_t send = b3 ? v[j] : v[j + 2], mine = b3 ? v[j + 2] : v[j];
    v[j] = max(mine, dpp_u32<kDppMirror>(send));
  }
  const bool b2 = lane & 4;
  const uint32_t send = b2 ? v[0] : v[1], mine = b2 ? v[1] : v[0];
  uint32_t m = max(mine, dpp_u32<kDppHalfMirror>(send));
  m = max(m, dpp_u32<kDppXor1>(m));
  return bits_f(max(m, dpp_u32<kDppXor2>(m)));
}

template <int D>
__device__ __forceinline__ uint32_t quantize_wave_vector(uint2 raw, float& scale) {
  float x[D / kWave];
  unpack_wave_vector<D>(raw, x);
  return quantize_wave_values<D>(x, scale);
}

// Rotary position embedding of one wave-held D-vector, rotate-half pairing
// over the first R dims ([KV] 2.2 names the step; the variant is the usual
// rotate-half one): for j < R/2, (x_j, x_{j+R/2}) turns by the angle whose
// cosine and sine are row[j] and row[R/2 + j]:
//   x_j' = x_j c - x_{j+R/2} s,   x_{j+R/2}' = x_{j+R/2} c + x_j s,
// each product and the sum / difference rounded to fp32 (no fused
// multiply-add).  Needs R % (2 D/64) == 0, so that the partner of a lane's
// element i is element i of the lane R/(2 D/64) further on.  Every lane of
// the wave must call it (the partner exchange is a wave permute).
template <int D>
__device__ __forceinline__ void rope_wave_vector(float (&x)[D / kWave], int lane, const float* row,
                                                 int R) {
#pragma clang fp contract(off)
  constexpr int EPL = D / kWave;
  const int hl = R / (2 * EPL);  // lanes that hold the first half
  const bool lower = lane < hl;
  const bool upper = !lower && lane < 2 * hl;
  const int partner = lower ? lane + hl : (upper ? lane - hl : lane);
  float p[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) p[i] = __shfl(x[i], partner, kWave);
  if (lower || upper) {
    const int j0 = (lower ? lane : lane - hl) * EPL;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const float c = row[j0 + i], sn = row[R / 2 + j0 + i];
      const float a = x[i] * c, b = p[i] * sn;
      x[i] = lower ? a - b : a + b;
    }
  }
}

// The same rotation over the whole head (R = D), with the token's table row
// already in registers as loaded by lanes in order: lane l holds row entries
// D/64 l .. D/64 l + D/64 - 1, i.e. the cosines of lanes 0-31 and the sines
// of lanes 32-63 for the same pair index.  Element i of lane l pairs with
// element i of lane l ^ 32, so one v_permlane32_swap per register gives each
// lane both its partner's element and the cosine and sine of its pair.
template <int D>
__device__ __forceinline__ void rope_wave_vector_full(float (&x)[D / kWave], int lane,
                                                      const float (&cs)[D / kWave]) {
#pragma clang fp contract(off)
  constexpr int EPL = D / kWave;
  const bool lower = lane < 32;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    uint32_t lo, hi, c, sn;
    swap32(f_bits(x[i]), lo, hi);      // lo: element of lane l % 32, hi: of lane l % 32 + 32
    swap32(f_bits(cs[i]), c, sn);      // c: cosine, sn: sine of the pair
    const float p = bits_f(lower ? hi : lo);
    const float a = x[i] * bits_f(c), b = p * bits_f(sn);
    x[i] = lower ? a - b : a + b;
  }
}

// The lane's D/64 bf16 elements of a D-vector (see quantize_wave_vector).
// NT: non-temporal loads (read-once inputs of the producer: the 2242- and
// 4096-token chunks measured 5-8% faster); the fused decode step reads its one
// new token with ordinary loads (the streaming hint measured slightly slower).
template <int D, bool NT = false>
__device__ __forceinline__ uint2 load_wave_vector(const uint16_t* src, int lane) {
  constexpr int EPL = D / kWave;
  typedef uint32_t v2u_ __attribute__((ext_vector_type(2)));
  if constexpr (EPL == 4) {
    const v2u_* p = reinterpret_cast<const v2u_*>(src + lane * 4);
    const v2u_ v = NT ? __builtin_nontemporal_load(p) : *p;
    return make_uint2(v[0], v[1]);
  } else if constexpr (EPL == 2) {
    const uint32_t* p = reinterpret_cast<const uint32_t*>(src + lane * 2);
    return make_uint2(NT ? __builtin_nontemporal_load(p) : *p, 0u);
  } else {
    return make_uint2((uint32_t)(NT ? __builtin_nontemporal_load(src + lane) : src[lane]), 0u);
  }
}

// Stores of one quantized token into the paged caches (lane's D/64 codes):
// K [blk, h, d/16, off, d%16] -- the lane's bytes sit in one 16-byte chunk;
// V [blk, h, d, off] -- one byte per (dim, token).
template <int D>
__device__ __forceinline__ void store_k_token(int8_t* k_cache, int64_t blk, int h, int Hkv, int off,
                                              int lane, uint32_t packed) {
  constexpr int EPL = D / kWave;
  const int d0 = lane * EPL;
  int8_t* dst = k_cache + (((blk * Hkv + h) * (D / 16) + d0 / 16) * kBlockSize + off) * 16 + d0 % 16;
  if constexpr (EPL == 4) *reinterpret_cast<uint32_t*>(dst) = packed;
  else if constexpr (EPL == 2) *reinterpret_cast<uint16_t*>(dst) = (uint16_t)packed;
  else *dst = (int8_t)packed;
}
template <int D>
__device__ __forceinline__ void store_v_token(int8_t* v_cache, int64_t blk, int h, int Hkv, int off,
                                              int lane, uint32_t packed) {
  constexpr int EPL = D / kWave;
  const int d0 = lane * EPL;
  int8_t* dst = v_cache + ((blk * Hkv + h) * D + d0) * kBlockSize + off;
#pragma unroll
  for (int i = 0; i < EPL; ++i) dst[i * kBlockSize] = (int8_t)(packed >> (8 * i));
}

}  // namespace i8kv
