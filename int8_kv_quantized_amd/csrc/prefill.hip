// Chunked prefill with history over the INT8 KV cache: one online softmax
// over the history pages and the causal chunk.
//
// What is computed follows the page "Implementing INT8 PV MMAC on a gfx936
// DCU: V-scale fusion, probability quantization, fragment grouping":
//   section 2   score = acc * sQ * sK / sqrt(d);
//   section 2.1 state (m, l, o): m' = max(m, max s), alpha = exp(m - m'),
//               p~ = exp(s - m'), W = p~ * sV quantized per G-key group,
//               o = alpha o + sum sW (Wq x Vq), l = alpha l + sum p~, O = o / l;
//   section 3/4 W and V are the two int8 operands of the PV product; one
//               scale per group of exactly the keys one MFMA (chain) consumes;
// and "INT8 KV and INT8 MMAC attention inference optimisation on a gfx936
// DCU", section 3.2 (history and chunk in the same online softmax) and
// section 4.2 (many query rows per workgroup so each K/V tile is reused).
//
// gfx950 mapping.  A workgroup of 12 waves owns 192 consecutive flattened
// rows (query token, q head of the GQA group) of one (sequence, KV head) --
// 32 tokens x 6 heads for 24 q heads over 4 KV heads; wave w owns 16 rows and lane
// l row l%16 (the four lanes l%16 + 16j share a row).  K/V tiles of 64 keys
// are staged in LDS in their page layouts.
//  * Tiles go from HBM straight into LDS (global_load_lds_dwordx4: one wave
//    instruction moves 1 KiB, lane l landing at +16 l), double-buffered: the
//    loads of tile t+1 are in flight while tile t is computed.  The source
//    address of each lane is free, so the K tile is permuted inside every
//    1 KiB piece while it is copied (see k_lds_off).
//  * QK, transposed: S^T = K Q^T with v_mfma_i32_16x16x64_i8 (operand A = 16
//    keys x 64 head-dim bytes from LDS, operand B = the int8 queries held in
//    registers).  Two MFMA chains per 32-key group; their A rows read keys
//    8(r/4) + 4b + r%4, so output register i of lane l in chain b is key
//    8(l/16) + 4b + i: each lane ends with 8 consecutive keys of its row.
//  * PV, also transposed: O^T = V^T Wq^T with v_mfma_i32_16x16x32_i8 (K = 32
//    keys = one group for G = 32; two chained MFMAs for G = 64).  Operand B
//    is Wq^T, whose lane slice is exactly the 8 keys the lane already holds;
//    operand A is V^T, 8 tokens of one dim from the LDS copy of the page.  The
//    output O^T keeps lane l on row l%16, so sW, alpha and l are per-lane
//    scalars and the group rescale O += sW * float(C) needs no exchange.
//    For G = 32 the MFMA accumulator starts at a bias that makes its int32
//    result readable as fp32 without a conversion, and the two groups of a
//    tile are folded into O with three VALU operations per element instead
//    of four (see the PV step).
//  * Online softmax in base 2 (log2 e folded into the per-row constant);
//    the output is rescaled only when the running max grows by more than 8
//    (p~ stays below 2^8), which is exact in real arithmetic since Wq and O
//    do not depend on the reference max.
#include <type_traits>

#include "device_common.hpp"
#include "kernels.hpp"

namespace i8kv {

namespace {

constexpr int kKT = 64;            // keys per tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazy = 8.0f;      // rescale threshold (log2 units)
constexpr float kMagic = 12582912.0f;      // 1.5 * 2^23
constexpr int kMagicBits = 0x4B400000;     // its fp32 bit pattern
constexpr int kPvAhead = 2;               // PV: V operands read this many 16-dim tiles ahead

// Reduce over the four lanes that share a row (lanes r, r+16, r+32, r+48).
__device__ __forceinline__ float row_max4(float v) {
  uint32_t a, b;
  swap16(f_bits(v), a, b);
  v = fmaxf(bits_f(a), bits_f(b));
  swap32(f_bits(v), a, b);
  return fmaxf(bits_f(a), bits_f(b));
}
// Maxima of two non-negative values over the four lanes of a row: integer
// max on the bit patterns (non-negative floats order like their bits, so no
// NaN quieting is needed), one reduce-scatter for both values -- after the
// first swap each 16-lane row holds one value's pair maximum -- and one more
// swap that hands every lane both results.
__device__ __forceinline__ void row_max4_pair_nonneg(float x0, float x1, float& m0, float& m1) {
  auto r = __builtin_amdgcn_permlane16_swap(f_bits(x0), f_bits(x1), false, false);
  uint32_t m = max((uint32_t)r[0], (uint32_t)r[1]);
  r = __builtin_amdgcn_permlane32_swap(m, m, false, false);
  m = max((uint32_t)r[0], (uint32_t)r[1]);
  r = __builtin_amdgcn_permlane16_swap(m, m, false, false);
  m0 = bits_f(r[0]);
  m1 = bits_f(r[1]);
}
__device__ __forceinline__ float row_sum4(float v) {
  uint32_t a, b;
  swap16(f_bits(v), a, b);
  v = bits_f(a) + bits_f(b);
  swap32(f_bits(v), a, b);
  return bits_f(a) + bits_f(b);
}

}  // namespace

// LDS layout of a K tile (4 pages of 16 keys): page j at j*(D*16 + 128), so odd
// pages start 128 bytes into a 256-byte bank row; inside a page, 16-byte chunk
// ch (head-dim bytes 16ch..16ch+15)
// of all 16 keys at ch*256, key kp at slot kperm(kp).  kperm swaps keys 8..11
// and 12..15 (an involution).  The 16 keys one QK operand read touches -- keys
// {4b..4b+3, 8+4b..11+4b} of two consecutive pages -- then fill all sixteen
// 16-byte slots of a 256-byte bank row, so the read has no bank conflict (the
// previous padded layout measured two-way conflicts).
__device__ __forceinline__ int kperm(int kp) { return kp ^ ((kp >> 3) << 2); }

template <int D>
__device__ __forceinline__ int k_lds_off(int key) {  // offset of chunk 0 of `key`
  return (key >> 4) * (D * 16 + 128) + 16 * kperm(key & 15);
}

// Waves per workgroup (16 flattened rows each): 12; 8 for the BF16-QK
// ablation, whose bf16 queries take twice the registers.
template <bool QB>
struct PrefillShape {
  static constexpr int NW = QB ? 8 : 12;
  static constexpr int Rows = 16 * NW;
};

// BF16-QK: the K tile converted to bf16, one row of D values per key plus 8
// values of padding; within each 32-key group the keys of QK chain b sit at
// rows 16b .. 16b + 15 in the order of the MFMA's A rows, so the 16 lanes of
// one operand read consecutive rows (no bank conflict).
template <int D>
struct PrefillKb {
  static constexpr int Pitch = D + 8;  // bf16 elements per row
  __device__ static int row(int key) {  // key = 32g + 8q + 4b + i -> 32g + 16b + 4q + i
    return (key & ~31) + 16 * ((key >> 2) & 1) + 4 * ((key >> 3) & 3) + (key & 3);
  }
};

template <int D>
struct PrefillTile {
  static constexpr int kBytes = kKT / 16 * (D * 16 + 128);  // K tile (pages 128 B apart)
  static constexpr int vBytes = kKT / 16 * D * 16;        // V tile [page][dim][16]
  static constexpr int kPieces = kKT / 16 * D * 16 / 1024;  // 1 KiB pieces per operand
  static constexpr int kPagePieces = D * 16 / 1024;         // pieces per page
};

// BPV: the BF16-PV ablation -- W = p~ sV rounded to bf16 (no W groups) times
// the int8 V taken exactly as bf16, v_mfma_f32_16x16x32_bf16 accumulating
// straight into O; the output is rescaled at every growth of the running max
// (as the per-tile reference of the online softmax), since bf16 rounding,
// unlike the group quantization, depends on the reference.
// QB: the BF16-QK ablation -- the bf16 queries (not quantized) against the
// int8 K codes taken exactly as bf16: each K tile, once landed, is converted
// to bf16 in LDS by the whole workgroup, and S^T = K Q^T runs on
// v_mfma_f32_16x16x32_bf16 with fp32 accumulation; score = dot * sK * scale.
// U8W: UINT8 W groups (sW = max W / 255, codes 0..255 passed to the signed
// MFMA as c - 128; a second MFMA against all-ones gives each group's sum of V,
// and 128 times it is added back in int32, exactly).
template <int D, int G, bool BPV, bool QB, bool U8W = false>
__global__ __launch_bounds__(PrefillShape<QB>::NW * kWave) void prefix_prefill_kernel(
    PrefillArgs a) {
  constexpr int kNW = PrefillShape<QB>::NW;
  constexpr int kRows = PrefillShape<QB>::Rows;
  constexpr int NC = D / 64;   // 64-dim k-steps of QK
  constexpr int NN = D / 16;   // 16-dim output tiles of PV
  constexpr int NT = kNW * kWave;
  constexpr int KBP = PrefillKb<D>::Pitch;
  constexpr int KB = PrefillTile<D>::kBytes, VB = PrefillTile<D>::vBytes;
  constexpr int NPC = PrefillTile<D>::kPieces, PPP = PrefillTile<D>::kPagePieces;
  constexpr int kMaxBt = 4096;                    // block-table entries kept in LDS

  __shared__ __attribute__((aligned(16))) int8_t s_k[2][KB];
  __shared__ __attribute__((aligned(16))) int8_t s_v[2][VB];
  __shared__ __attribute__((aligned(16))) float s_sk[2][kKT];
  __shared__ __attribute__((aligned(16))) float s_sv[2][kKT];
  __shared__ int s_bt[kMaxBt];
  __shared__ __attribute__((aligned(16))) uint16_t s_kb[QB ? kKT * KBP : 8];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int lg = lane >> 4, lr = lane & 15;
  const int s = blockIdx.z, kv = blockIdx.y;
  const int grp = a.group, Hkv = a.num_kv_heads;

  const int q0 = a.query_start_loc[s];
  const int chunk = a.query_start_loc[s + 1] - q0;
  const int seq_len = a.seq_lens[s];
  const int ctx = seq_len - chunk;
  const int nrows_seq = chunk * grp;
  const int row0 = blockIdx.x * kRows;
  if (row0 >= nrows_seq || ctx < 0) return;

  // this lane's row
  const int fr = row0 + 16 * w + lr;
  const bool row_ok = fr < nrows_seq;
  const int tok = row_ok ? fr / grp : 0;
  const int head = row_ok ? fr % grp : 0;
  const int pos = ctx + tok;
  const size_t qrow = (size_t)(q0 + tok) * a.num_q_heads + (size_t)kv * grp + head;

  v4i qb[QB ? 1 : NC];
  v4u qh[QB ? NC : 1][2];  // QB: bf16 dims 64c + 16lg + 8e .. +7 of this lane's row
  if constexpr (QB) {
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int e = 0; e < 2; ++e)
        qh[c][e] = row_ok ? *reinterpret_cast<const v4u*>(a.q_bf16 + qrow * D + 64 * c +
                                                          16 * lg + 8 * e)
                          : v4u{0u, 0u, 0u, 0u};
  } else {
#pragma unroll
    for (int c = 0; c < NC; ++c)
      qb[c] = row_ok ? *reinterpret_cast<const v4i*>(a.q_int8 + qrow * D + 64 * c + 16 * lg)
                     : v4i{0, 0, 0, 0};
  }
  // score in log2 units: s2 = acc * sK * (sQ * softmax_scale * log2 e) (QB:
  // s2 = dot * sK * (softmax_scale * log2 e)).  A row past the chunk gets
  // crow = 1 and mref = +inf, which makes all its p~ zero without a select
  // (its queries are zero, so its scores are 0 or -inf).
  const float crow =
      row_ok ? (QB ? 1.0f : a.q_scale[qrow]) * a.softmax_scale * kLog2e : 1.0f;

  const int last_fr = min(row0 + kRows, nrows_seq) - 1;
  const int nkeys = ctx + last_fr / grp + 1;  // keys visible to the workgroup's last row
  const int wave_first_fr = row0 + 16 * w;
  const int wave_last_fr = min(wave_first_fr + 15, nrows_seq - 1);
  const bool wave_live = wave_first_fr < nrows_seq;
  const int wave_nkeys = wave_live ? ctx + wave_last_fr / grp + 1 : 0;
  const int wave_min_pos = wave_live ? ctx + wave_first_fr / grp : 0;
  const int ntiles = (nkeys + kKT - 1) / kKT;
  const int npages_seq = min((seq_len + kBlockSize - 1) / kBlockSize, a.max_blocks_per_seq);
  const int npages_used = min((nkeys + kBlockSize - 1) / kBlockSize, npages_seq);
  const bool bt_in_lds = npages_used <= kMaxBt;
  const int32_t* bt_row = a.block_tables + (size_t)s * a.max_blocks_per_seq;
  if (bt_in_lds)
    for (int i = tid; i < npages_used; i += NT)
      s_bt[i] = min(max(bt_row[i], 0), a.num_blocks - 1);
  __syncthreads();
  // Page id of page pg of the sequence; pages past the keys in use map to page
  // 0 of the cache (their keys are masked: score -inf, W 0).
  auto page_id = [&](int pg) -> int {
    if (pg >= npages_used) return 0;
    return bt_in_lds ? s_bt[pg] : min(max(bt_row[pg], 0), a.num_blocks - 1);
  };

  // ---- tile loads: HBM -> LDS directly -----------------------------------------
  // Wave w copies pieces w, w + kNW, ... of the 2 * NPC 1 KiB pieces of a tile
  // (K pieces first, then V); the last two waves also copy the 64 K and V
  // scales.  Lane l of a K piece fetches the key that belongs at slot l & 15.
  // The pieces a wave copies are the same for every tile: their page in the
  // tile, LDS offset and per-lane source offset are set up once (wave-uniform
  // except the lane offset); per tile only the page id changes.
  constexpr int kMaxPieces = (2 * NPC + kNW - 1) / kNW;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const int koff_lane = (lane >> 4) * 256 + kperm(lane & 15) * 16;
  int pc_j[kMaxPieces], pc_lds[kMaxPieces], pc_src[kMaxPieces];
  bool pc_v[kMaxPieces];
#pragma unroll
  for (int i = 0; i < kMaxPieces; ++i) {
    const int q = min(wu + i * kNW, 2 * NPC - 1);
    pc_v[i] = q >= NPC;
    const int qq = pc_v[i] ? q - NPC : q;
    const int cp = qq % PPP;
    pc_j[i] = qq / PPP;
    pc_lds[i] = pc_v[i] ? pc_j[i] * D * 16 + cp * 1024 : pc_j[i] * (D * 16 + 128) + cp * 1024;
    pc_src[i] = cp * 1024 + (pc_v[i] ? lane * 16 : koff_lane);
  }
  auto issue_tile = [&](int t, int buf) {
    const int k0 = t * kKT;
#pragma unroll
    for (int i = 0; i < kMaxPieces; ++i) {
      if (wu + i * kNW >= 2 * NPC) break;  // wave-uniform
      const int pid = __builtin_amdgcn_readfirstlane(page_id(k0 / kBlockSize + pc_j[i]));
      const int8_t* src = (pc_v[i] ? a.v_cache : a.k_cache) +
                          ((size_t)pid * Hkv + kv) * (size_t)D * 16 + pc_src[i];
      int8_t* dst = (pc_v[i] ? s_v[buf] : s_k[buf]) + pc_lds[i];
      __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)dst, 16, 0,
                                       0);
    }
    if (w >= kNW - 2) {  // scale of key k0 + lane (keys past the sequence: any finite
                         // or not value, discarded by the masked path)
      const int pid = page_id((k0 + lane) / kBlockSize);
      const size_t idx = ((size_t)pid * kBlockSize + (lane % 16)) * Hkv + kv;
      if (w == kNW - 1)
        __builtin_amdgcn_global_load_lds(a.k_scale + idx,
                                         (__attribute__((address_space(3))) void*)s_sk[buf], 4, 0, 0);
      else
        __builtin_amdgcn_global_load_lds(a.v_scale + idx,
                                         (__attribute__((address_space(3))) void*)s_sv[buf], 4, 0, 0);
    }
  };
  // every copy of this wave has landed in LDS (the barrier that follows makes
  // all waves' copies visible)
  auto wait_tile = [&]() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };
  // QB: K tile `buf` (landed and visible) -> bf16 rows of s_kb; unit u is the
  // 16 head-dim bytes of chunk u / 64 of key u % 64.  A barrier must follow.
  auto convert_k = [&](int buf) {
    for (int u = tid; u < kKT * (D / 16); u += NT) {
      const int key = u & (kKT - 1), ch = u / kKT;
      const v4u kw = *reinterpret_cast<const v4u*>(s_k[buf] + k_lds_off<D>(key) + 256 * ch);
      uint16_t* dst = s_kb + PrefillKb<D>::row(key) * KBP + 16 * ch;
      *reinterpret_cast<v8bf*>(dst) = i8x8_to_bf16(kw[0], kw[1]);
      *reinterpret_cast<v8bf*>(dst + 8) = i8x8_to_bf16(kw[2], kw[3]);
    }
  };

  float mref = row_ok ? -INFINITY : INFINITY;  // reference max (log2 units)
  float lsum = 0.0f;                           // this lane's share of l
  float rc = 0.0f;                             // G = 32: offset carried by O (per row)
  const v4i mag4 = {kMagicBits, kMagicBits, kMagicBits, kMagicBits};
  float O[NN][4];
#pragma unroll
  for (int n = 0; n < NN; ++n)
#pragma unroll
    for (int i = 0; i < 4; ++i) O[n][i] = 0.0f;

  // One 64-key tile from LDS buffer `buf`; MASK: keys past a row's position
  // may be present (diagonal tiles only).
  auto compute_tile = [&](int buf, int k0, auto mask_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const int8_t* kt = s_k[buf];
    // ---- S^T = K Q^T: per 32-key group g, two chains of D/64 MFMAs -------
    float u2[2][8];
    float mt = -INFINITY;
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      v4i acc[2];
      v4f accf[QB ? 2 : 1];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        if constexpr (QB) {
          // A row lr = key 32g + 8(lr/4) + 4b + lr%4, stored at row 32g + 16b + lr
          const uint16_t* kp = s_kb + (32 * g + 16 * b + lr) * KBP + 16 * lg;
          accf[b] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int c = 0; c < NC; ++c)
#pragma unroll
            for (int e = 0; e < 2; ++e) {
              const v8bf ka = *reinterpret_cast<const v8bf*>(kp + 64 * c + 8 * e);
              accf[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                  ka, __builtin_bit_cast(v8bf, qh[c][e]), accf[b], 0, 0, 0);
            }
        } else {
          acc[b] = v4i{0, 0, 0, 0};
          const int krow = 32 * g + 8 * (lr >> 2) + 4 * b + (lr & 3);  // key of A row lr
          const int8_t* kp = kt + k_lds_off<D>(krow) + 256 * lg;
#pragma unroll
          for (int c = 0; c < NC; ++c) {
            const v4i ka = *reinterpret_cast<const v4i*>(kp + 1024 * c);
            acc[b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(ka, qb[c], acc[b], 0, 0, 0);
          }
        }
      }
      const float4 sk0 = *reinterpret_cast<const float4*>(&s_sk[buf][32 * g + 8 * lg]);
      const float4 sk1 = *reinterpret_cast<const float4*>(&s_sk[buf][32 * g + 8 * lg + 4]);
      const float skv[8] = {sk0.x, sk0.y, sk0.z, sk0.w, sk1.x, sk1.y, sk1.z, sk1.w};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float x = (QB ? accf[j >> 2][j & 3] : (float)acc[j >> 2][j & 3]) * skv[j];
        if constexpr (MASK) x = (k0 + 32 * g + 8 * lg + j <= pos) ? x : -INFINITY;
        u2[g][j] = x;
        mt = fmaxf(mt, x);
      }
    }
    // ---- online softmax (base 2, lazy rescale) -------------------------------
    mt = row_max4(mt) * crow;
    const bool grow = row_ok && mt != -INFINITY && (mt > mref + (BPV ? 0.0f : kLazy) || mref == -INFINITY);
    if (__builtin_amdgcn_ballot_w64(grow)) {
      const float alpha = grow ? (mref == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mref - mt))
                               : 1.0f;
      if (grow) mref = mt;
      lsum *= alpha;
      rc *= alpha;
#pragma unroll
      for (int n = 0; n < NN; ++n)
#pragma unroll
        for (int i = 0; i < 4; ++i) O[n][i] *= alpha;
    }
    // p~ = 2^(s2 - mref), W = p~ sV, Wq = round(W * 127 / max W)
    uint32_t wpk[2][2];
    float swg[2], am[2], mxg[2], Wv[2][8];
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const float4 sv0 = *reinterpret_cast<const float4*>(&s_sv[buf][32 * g + 8 * lg]);
      const float4 sv1 = *reinterpret_cast<const float4*>(&s_sv[buf][32 * g + 8 * lg + 4]);
      const float svv[8] = {sv0.x, sv0.y, sv0.z, sv0.w, sv1.x, sv1.y, sv1.z, sv1.w};
      float mx = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float pt = __builtin_amdgcn_exp2f(__builtin_fmaf(u2[g][j], crow, -mref));
        Wv[g][j] = pt * svv[j];
        if constexpr (MASK) {
          // a masked key has p~ = 0 and W = 0 whatever its score constant
          // (crow = 0 for an all-zero query) or scale (any value past the
          // sequence) would give
          const bool vis = k0 + 32 * g + 8 * lg + j <= pos;
          pt = vis ? pt : 0.0f;
          Wv[g][j] = vis ? Wv[g][j] : 0.0f;
        }
        lsum += pt;
        mx = fmaxf(mx, Wv[g][j]);
      }
      mxg[g] = mx;
    }
    row_max4_pair_nonneg(mxg[0], mxg[1], am[0], am[1]);
    if constexpr (BPV) {
      // ---- O^T += V^T W^T in bf16 (keys of group g: the lane's 8 W values)
      const int8_t* vt = s_v[buf];
      const int voff = 8 * (lg & 1);
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        v4u wu;
#pragma unroll
        for (int k = 0; k < 4; ++k)
          wu[k] = bf16_rne_bits(Wv[g][2 * k]) | (bf16_rne_bits(Wv[g][2 * k + 1]) << 16);
        const v8bf wb = __builtin_bit_cast(v8bf, wu);
        const int8_t* vp = vt + ((2 * g + (lg >> 1)) * D + lr) * 16 + voff;
#pragma unroll
        for (int n = 0; n < NN; ++n) {
          const uint2 vv = *reinterpret_cast<const uint2*>(vp + 256 * n);
          v4f c = v4f{O[n][0], O[n][1], O[n][2], O[n][3]};
          c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(i8x8_to_bf16(vv.x, vv.y), wb, c, 0, 0, 0);
#pragma unroll
          for (int i = 0; i < 4; ++i) O[n][i] = c[i];
        }
      }
      return;
    }
    if constexpr (G == 64) am[0] = am[1] = fmaxf(am[0], am[1]);
    constexpr float kQmax = U8W ? 255.0f : 127.0f;
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      swg[g] = am[g] * (1.0f / kQmax);
      // inv = kQmax / max W (hardware reciprocal, within an ulp); the code is
      // W * inv rounded to the nearest integer by the byte conversion itself
      // (nearest-even on an exact tie, saturating at 255, so W <= max W stays
      // in [0, kQmax]): one instruction per code for the multiply and one for
      // round-and-pack
      const float inv = am[g] > 0.0f ? kQmax * __builtin_amdgcn_rcpf(am[g]) : 0.0f;
      uint32_t pk[2] = {0, 0};
#pragma unroll
      for (int j = 0; j < 8; ++j)
        pk[j >> 2] = __builtin_amdgcn_cvt_pk_u8_f32(Wv[g][j] * inv, j & 3, pk[j >> 2]);
      wpk[g][0] = U8W ? pk[0] ^ 0x80808080u : pk[0];  // UINT8: c - 128 as int8
      wpk[g][1] = U8W ? pk[1] ^ 0x80808080u : pk[1];
    }
    // ---- O^T += sW * (V^T Wq^T) --------------------------------------------------
    const int8_t* vt = s_v[buf];
    const int voff = 8 * (lg & 1);
    if constexpr (U8W) {
      // per group: C = V^T (Wq - 128)^T, CS = V^T 1 (the group's sum of V per
      // dim, the same for every row), O += sW * float(C + 128 CS)
      const long ones8 = 0x0101010101010101L;
      const v4i ones16 = {0x01010101, 0x01010101, 0x01010101, 0x01010101};
      const long wb0 = (long)(((uint64_t)wpk[0][1] << 32) | wpk[0][0]);
      const long wb1 = (long)(((uint64_t)wpk[1][1] << 32) | wpk[1][0]);
      const v4i wb = {(int)wpk[0][0], (int)wpk[0][1], (int)wpk[1][0], (int)wpk[1][1]};
      const int8_t* vp0 = vt + ((lg >> 1) * D + lr) * 16 + voff;
      const int8_t* vp1 = vt + ((2 + (lg >> 1)) * D + lr) * 16 + voff;
      const v4i z = {0, 0, 0, 0};
#pragma unroll
      for (int n = 0; n < NN; ++n) {
        const long va0 = *reinterpret_cast<const long*>(vp0 + 256 * n);
        const long va1 = *reinterpret_cast<const long*>(vp1 + 256 * n);
        if constexpr (G == 32) {
          const v4i c0 = __builtin_amdgcn_mfma_i32_16x16x32_i8(va0, wb0, z, 0, 0, 0);
          const v4i c1 = __builtin_amdgcn_mfma_i32_16x16x32_i8(va1, wb1, z, 0, 0, 0);
          const v4i s0 = __builtin_amdgcn_mfma_i32_16x16x32_i8(va0, ones8, z, 0, 0, 0);
          const v4i s1 = __builtin_amdgcn_mfma_i32_16x16x32_i8(va1, ones8, z, 0, 0, 0);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            O[n][i] = __builtin_fmaf(swg[0], (float)(c0[i] + (s0[i] << 7)), O[n][i]);
            O[n][i] = __builtin_fmaf(swg[1], (float)(c1[i] + (s1[i] << 7)), O[n][i]);
          }
        } else {
          const v4i va = {(int)(uint32_t)va0, (int)(uint32_t)((uint64_t)va0 >> 32),
                          (int)(uint32_t)va1, (int)(uint32_t)((uint64_t)va1 >> 32)};
          const v4i c = __builtin_amdgcn_mfma_i32_16x16x64_i8(va, wb, z, 0, 0, 0);
          const v4i cs = __builtin_amdgcn_mfma_i32_16x16x64_i8(va, ones16, z, 0, 0, 0);
#pragma unroll
          for (int i = 0; i < 4; ++i)
            O[n][i] = __builtin_fmaf(swg[0], (float)(c[i] + (cs[i] << 7)), O[n][i]);
        }
      }
    } else if constexpr (G == 32) {
      // Both groups of the tile in one pass, the int32 -> fp32 conversion done
      // by the MFMA: its accumulator starts at the bit pattern of kMagic, so
      // the result read as fp32 is exactly kMagic + acc (|acc| <= 32 * 127^2 <
      // 2^22 keeps it inside the binade [2^23, 2^24), where one unit of the
      // bit pattern is 1.0).  With sW cut to 22 significant bits (a relative
      // change below 2^-21) the products P_g = kMagic * sW_g are exact, and
      //   fma(sW1, x1, fma(sW0, x0, -S)) = sW0 acc0 + sW1 acc1 + d,
      // S = fl(P0 + P1), d = P0 + P1 - S exactly (Fast2Sum, P_g >= 0); d is
      // per row and is taken off once at the end (rc).  The one rounding left
      // per element is that of the inner fma, whose value is about -P1:
      // at most ~sW1 / 2^1, i.e. under one unit of a single Wq * Vq product.
      const float sw0 = bits_f(f_bits(swg[0]) & ~3u), sw1 = bits_f(f_bits(swg[1]) & ~3u);
      const float p0 = kMagic * sw0, p1 = kMagic * sw1;
      const float ph = fmaxf(p0, p1), pl = fminf(p0, p1);
      const float S = ph + pl;
      rc += pl - (S - ph);
      const float nS = -S;
      const long wb0 = (long)(((uint64_t)wpk[0][1] << 32) | wpk[0][0]);
      const long wb1 = (long)(((uint64_t)wpk[1][1] << 32) | wpk[1][0]);
      const int8_t* vp0 = vt + ((lg >> 1) * D + lr) * 16 + voff;
      const int8_t* vp1 = vt + ((2 + (lg >> 1)) * D + lr) * 16 + voff;
      // V operands read kPvAhead 16-dim tiles ahead of their MFMAs, so the
      // LDS latency is not on each MFMA's path (2 measured 3% faster than the
      // compiler's own order; 4 and 6 less)
      constexpr int PD = kPvAhead;
      long ra0[PD], ra1[PD];
#pragma unroll
      for (int q = 0; q < PD; ++q) {
        ra0[q] = *reinterpret_cast<const long*>(vp0 + 256 * q);
        ra1[q] = *reinterpret_cast<const long*>(vp1 + 256 * q);
      }
#pragma unroll
      for (int n = 0; n < NN; ++n) {
        const long va0 = ra0[n % PD], va1 = ra1[n % PD];
        if (n + PD < NN) {
          ra0[n % PD] = *reinterpret_cast<const long*>(vp0 + 256 * (n + PD));
          ra1[n % PD] = *reinterpret_cast<const long*>(vp1 + 256 * (n + PD));
        }
        const v4i c0 = __builtin_amdgcn_mfma_i32_16x16x32_i8(va0, wb0, mag4, 0, 0, 0);
        const v4i c1 = __builtin_amdgcn_mfma_i32_16x16x32_i8(va1, wb1, mag4, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          O[n][i] += __builtin_fmaf(sw1, bits_f((uint32_t)c1[i]),
                                    __builtin_fmaf(sw0, bits_f((uint32_t)c0[i]), nS));
      }
    } else {
      // G = 64: the whole tile is one group, consumed by one K = 64 MFMA per
      // 16-dim tile (gfx950's full-rate int8 shape; two chained K = 32 ones
      // take twice the matrix-core cycles).  The lane's 16 bytes of operand B
      // are its 8 keys of each half (8(l/16) .. +7 and 32 + 8(l/16) .. +7), and
      // operand A carries V of the same 16 keys in the same byte positions, so
      // the product sums exactly the tile's 64 keys.
      const v4i wb = {(int)wpk[0][0], (int)wpk[0][1], (int)wpk[1][0], (int)wpk[1][1]};
      const int8_t* vp0 = vt + ((lg >> 1) * D + lr) * 16 + voff;
      const int8_t* vp1 = vt + ((2 + (lg >> 1)) * D + lr) * 16 + voff;
      constexpr int PD = kPvAhead;
      uint2 ra0[PD], ra1[PD];
#pragma unroll
      for (int q = 0; q < PD; ++q) {
        ra0[q] = *reinterpret_cast<const uint2*>(vp0 + 256 * q);
        ra1[q] = *reinterpret_cast<const uint2*>(vp1 + 256 * q);
      }
#pragma unroll
      for (int n = 0; n < NN; ++n) {
        const uint2 va0 = ra0[n % PD], va1 = ra1[n % PD];
        if (n + PD < NN) {
          ra0[n % PD] = *reinterpret_cast<const uint2*>(vp0 + 256 * (n + PD));
          ra1[n % PD] = *reinterpret_cast<const uint2*>(vp1 + 256 * (n + PD));
        }
        const v4i va = {(int)va0.x, (int)va0.y, (int)va1.x, (int)va1.y};
        const v4i c = __builtin_amdgcn_mfma_i32_16x16x64_i8(va, wb, v4i{0, 0, 0, 0}, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) O[n][i] += swg[0] * (float)c[i];
      }
    }
  };

  issue_tile(0, 0);
  wait_tile();
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    const int k0 = t * kKT;
    if constexpr (QB) {
      convert_k(buf);
      __syncthreads();
    }
    if (t + 1 < ntiles) issue_tile(t + 1, buf ^ 1);  // in flight during this tile's compute
    if (k0 < wave_nkeys) {
      if (k0 + kKT - 1 > wave_min_pos) compute_tile(buf, k0, std::true_type{});
      else compute_tile(buf, k0, std::false_type{});
    }
    wait_tile();
    __syncthreads();
  }

  // ---- O / l and store: lane l holds row l%16, dims 16n + 4(l/16) + i ----------
  const float l_row = row_sum4(lsum);
  if (!row_ok) return;
  const float inv = 1.0f / l_row;
  if (a.out16) {  // the same fp32 values, rounded to bf16 (nearest, ties to even)
    uint16_t* dst = a.out16 + qrow * D + 4 * lg;
#pragma unroll
    for (int n = 0; n < NN; ++n)
      *reinterpret_cast<uint2*>(dst + 16 * n) =
          make_uint2(bf16_rne_bits((O[n][0] - rc) * inv) | (bf16_rne_bits((O[n][1] - rc) * inv) << 16),
                     bf16_rne_bits((O[n][2] - rc) * inv) | (bf16_rne_bits((O[n][3] - rc) * inv) << 16));
    return;
  }
  float* dst = a.out + qrow * D + 4 * lg;
#pragma unroll
  for (int n = 0; n < NN; ++n)
    *reinterpret_cast<float4*>(dst + 16 * n) =
        make_float4((O[n][0] - rc) * inv, (O[n][1] - rc) * inv, (O[n][2] - rc) * inv,
                    (O[n][3] - rc) * inv);
}

hipError_t launch_prefix_prefill(const PrefillArgs& a, hipStream_t stream) {
  if (a.num_seqs == 0 || a.max_query_len == 0) return hipSuccess;
  const int64_t rows = (int64_t)a.max_query_len * a.group;
  const bool qb = a.q_bf16 != nullptr;
  const int64_t per_wg = qb ? PrefillShape<true>::Rows : PrefillShape<false>::Rows;
  const int64_t tiles = (rows + per_wg - 1) / per_wg;
  dim3 grid((unsigned)tiles, (unsigned)a.num_kv_heads, (unsigned)a.num_seqs);
  dim3 block((qb ? PrefillShape<true>::NW : PrefillShape<false>::NW) * kWave);
#define I8KV_PREFILL_CASE(DD, GG)                                                              \
  if (a.head_dim == DD && (a.pv_bf16 ? GG == 64 : a.w_group == GG)) {                          \
    if (qb)                                                                                    \
      hipLaunchKernelGGL((prefix_prefill_kernel<DD, GG, false, true>), grid, block, 0, stream, \
                         a);                                                                   \
    else if (a.pv_bf16)                                                                        \
      hipLaunchKernelGGL((prefix_prefill_kernel<DD, GG, true, false>), grid, block, 0, stream, \
                         a);                                                                   \
    else if (a.w_uint8)                                                                        \
      hipLaunchKernelGGL((prefix_prefill_kernel<DD, GG, false, false, true>), grid, block, 0,  \
                         stream, a);                                                           \
    else                                                                                       \
      hipLaunchKernelGGL((prefix_prefill_kernel<DD, GG, false, false>), grid, block, 0,        \
                         stream, a);                                                           \
    return hipGetLastError();                                                                  \
  }
  I8KV_PREFILL_CASE(64, 32)
  I8KV_PREFILL_CASE(64, 64)
  I8KV_PREFILL_CASE(128, 32)
  I8KV_PREFILL_CASE(128, 64)
  I8KV_PREFILL_CASE(256, 32)
  I8KV_PREFILL_CASE(256, 64)
#undef I8KV_PREFILL_CASE
  return hipErrorInvalidValue;
}

}  // namespace i8kv
