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
// 32 tokens x 6 heads for Qwen-like 24/4 heads; wave w owns 16 rows and lane
// l row l%16 (the four lanes l%16 + 16j share a row).  K/V tiles of 64 keys
// are staged in LDS in their page layouts.
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
//  * Online softmax in base 2 (log2 e folded into the per-row constant);
//    the output is rescaled only when the running max grows by more than 8
//    (p~ stays below 2^8), which is exact in real arithmetic since Wq and O
//    do not depend on the reference max.
#include "device_common.hpp"
#include "kernels.hpp"

namespace i8kv {

namespace {

constexpr int kNW = 12;            // waves per workgroup
constexpr int kRows = 16 * kNW;    // flattened rows per workgroup
constexpr int kKT = 64;            // keys per tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazy = 8.0f;      // rescale threshold (log2 units)

// Reduce over the four lanes that share a row (lanes r, r+16, r+32, r+48).
__device__ __forceinline__ float row_max4(float v) {
  uint32_t a, b;
  swap16(f_bits(v), a, b);
  v = fmaxf(bits_f(a), bits_f(b));
  swap32(f_bits(v), a, b);
  return fmaxf(bits_f(a), bits_f(b));
}
__device__ __forceinline__ float row_sum4(float v) {
  uint32_t a, b;
  swap16(f_bits(v), a, b);
  v = bits_f(a) + bits_f(b);
  swap32(f_bits(v), a, b);
  return bits_f(a) + bits_f(b);
}

}  // namespace

template <int D, int G>
__global__ __launch_bounds__(kNW * kWave) void prefix_prefill_kernel(PrefillArgs a) {
  constexpr int NC = D / 64;   // 64-dim k-steps of QK
  constexpr int NN = D / 16;   // 16-dim output tiles of PV
  constexpr int NT = kNW * kWave;
  // LDS tiles in page layout: K [page][chunk][key][16 B], V [page][dim][16 B]
  __shared__ __attribute__((aligned(16))) int8_t s_k[kKT / 16][D / 16][16][16];
  __shared__ __attribute__((aligned(16))) int8_t s_v[kKT / 16][D][16];
  __shared__ __attribute__((aligned(16))) float s_sk[kKT];
  __shared__ __attribute__((aligned(16))) float s_sv[kKT];
  __shared__ int s_pid[kKT / 16];

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

  v4i qb[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c)
    qb[c] = row_ok ? *reinterpret_cast<const v4i*>(a.q_int8 + qrow * D + 64 * c + 16 * lg)
                   : v4i{0, 0, 0, 0};
  // score in log2 units: s2 = acc * sK * (sQ * softmax_scale * log2 e)
  const float crow = row_ok ? a.q_scale[qrow] * a.softmax_scale * kLog2e : 0.0f;

  const int last_fr = min(row0 + kRows, nrows_seq) - 1;
  const int nkeys = ctx + last_fr / grp + 1;  // keys visible to the workgroup's last row
  const int wave_first_fr = row0 + 16 * w;
  const int wave_last_fr = min(wave_first_fr + 15, nrows_seq - 1);
  const bool wave_live = wave_first_fr < nrows_seq;
  const int wave_nkeys = wave_live ? ctx + wave_last_fr / grp + 1 : 0;
  const int wave_min_pos = wave_live ? ctx + wave_first_fr / grp : 0;
  const int ntiles = (nkeys + kKT - 1) / kKT;
  const int npages_seq = min((seq_len + kBlockSize - 1) / kBlockSize, a.max_blocks_per_seq);

  float mref = -INFINITY;  // reference max (log2 units) of this row
  float lsum = 0.0f;       // this lane's share of l
  float O[NN][4];
#pragma unroll
  for (int n = 0; n < NN; ++n)
#pragma unroll
    for (int i = 0; i < 4; ++i) O[n][i] = 0.0f;

  for (int t = 0; t < ntiles; ++t) {
    const int k0 = t * kKT;
    __syncthreads();
    if (tid < kKT / 16) {
      const int pg = k0 / kBlockSize + tid;
      int pid = -1;
      if (pg < npages_seq) {
        pid = a.block_tables[(size_t)s * a.max_blocks_per_seq + pg];
        pid = min(max(pid, 0), a.num_blocks - 1);
      }
      s_pid[tid] = pid;
    }
    __syncthreads();
    // K and V pages of the tile: 4 x (D*16) bytes each, 16 bytes per thread-step
    constexpr int kUnits = kKT / 16 * D;  // 16-byte units per tile and operand
    for (int u = tid; u < 2 * kUnits; u += NT) {
      const int isv = u >= kUnits;
      const int uu = isv ? u - kUnits : u;
      const int i = uu / D, rem = uu % D;
      const int pid = s_pid[i];
      v4i val = {0, 0, 0, 0};
      const int8_t* src = (isv ? a.v_cache : a.k_cache) + ((size_t)pid * Hkv + kv) * (size_t)D * 16 +
                          (size_t)rem * 16;
      if (pid >= 0) val = *reinterpret_cast<const v4i*>(src);
      int8_t* dst = isv ? &s_v[i][rem][0] : &s_k[i][rem / 16][rem % 16][0];
      *reinterpret_cast<v4i*>(dst) = val;
    }
    if (tid < kKT) {
      const int key = k0 + tid;
      const int pid = s_pid[tid / 16];
      float skv = 0.0f, svv = 0.0f;
      if (pid >= 0 && key < seq_len) {
        const size_t idx = ((size_t)pid * kBlockSize + (tid % 16)) * Hkv + kv;
        skv = a.k_scale[idx];
        svv = a.v_scale[idx];
      }
      s_sk[tid] = skv;
      s_sv[tid] = svv;
    }
    __syncthreads();
    if (k0 >= wave_nkeys) continue;  // no key of this tile is visible to the wave
    const bool diag = k0 + kKT - 1 > wave_min_pos;  // some key may be masked

    // ---- S^T = K Q^T: per 32-key group g, two chains of D/64 MFMAs ---------
    float u2[2][8];  // [group][key 8lg + j]: acc * sK, -inf when masked
    float mt = -INFINITY;
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      v4i acc[2];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        acc[b] = v4i{0, 0, 0, 0};
        const int krow = 32 * g + 8 * (lr >> 2) + 4 * b + (lr & 3);  // key of A row lr
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const v4i ka =
              *reinterpret_cast<const v4i*>(&s_k[krow >> 4][4 * c + lg][krow & 15][0]);
          acc[b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(ka, qb[c], acc[b], 0, 0, 0);
        }
      }
      const float4 sk0 = *reinterpret_cast<const float4*>(&s_sk[32 * g + 8 * lg]);
      const float4 sk1 = *reinterpret_cast<const float4*>(&s_sk[32 * g + 8 * lg + 4]);
      const float skv[8] = {sk0.x, sk0.y, sk0.z, sk0.w, sk1.x, sk1.y, sk1.z, sk1.w};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float x = (float)acc[j >> 2][j & 3] * skv[j];
        if (diag) {
          const int key = k0 + 32 * g + 8 * lg + j;
          x = (row_ok && key <= pos) ? x : -INFINITY;
        }
        u2[g][j] = x;
        mt = fmaxf(mt, x);
      }
    }
    // ---- online softmax (base 2, lazy rescale) -----------------------------
    mt = row_max4(mt) * crow;  // crow > 0: max of the scaled scores
    if (!row_ok) mt = -INFINITY;
    const bool grow = mt > mref + kLazy || mref == -INFINITY;
    if (__builtin_amdgcn_ballot_w64(grow && mt != -INFINITY)) {
      const float mnew = (grow && mt != -INFINITY) ? mt : mref;
      const float alpha = (mref == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(mref - mnew);
      if (mnew != mref) {
        lsum *= alpha;
#pragma unroll
        for (int n = 0; n < NN; ++n)
#pragma unroll
          for (int i = 0; i < 4; ++i) O[n][i] *= alpha;
        mref = mnew;
      }
    }
    // p~ = 2^(s2 - mref), W = p~ sV, Wq = round(W * 127 / max W)
    uint32_t wpk[2][2];
    float swg[2];
    float am[2];
    float Wv[2][8];
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const float4 sv0 = *reinterpret_cast<const float4*>(&s_sv[32 * g + 8 * lg]);
      const float4 sv1 = *reinterpret_cast<const float4*>(&s_sv[32 * g + 8 * lg + 4]);
      const float svv[8] = {sv0.x, sv0.y, sv0.z, sv0.w, sv1.x, sv1.y, sv1.z, sv1.w};
      float mx = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float pt =
            row_ok ? __builtin_amdgcn_exp2f(__builtin_fmaf(u2[g][j], crow, -mref)) : 0.0f;
        lsum += pt;
        Wv[g][j] = pt * svv[j];
        mx = fmaxf(mx, Wv[g][j]);
      }
      am[g] = row_max4(mx);
    }
    if constexpr (G == 64) am[0] = am[1] = fmaxf(am[0], am[1]);
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      swg[g] = am[g] * (1.0f / 127.0f);
      const float inv = am[g] > 0.0f ? 127.0f * __builtin_amdgcn_rcpf(am[g]) : 0.0f;
      uint32_t pk[2] = {0, 0};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t q = min((uint32_t)__builtin_fmaf(Wv[g][j], inv, 0.5f), 127u);
        pk[j >> 2] |= q << (8 * (j & 3));
      }
      wpk[g][0] = pk[0];
      wpk[g][1] = pk[1];
    }
    // ---- O^T += sW * (V^T Wq^T) ------------------------------------------------
    const int vpage_off = 8 * (lg & 1);
    if constexpr (G == 32) {
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const long wb = (long)(((uint64_t)wpk[g][1] << 32) | wpk[g][0]);
        const int vpg = 2 * g + (lg >> 1);
#pragma unroll
        for (int n = 0; n < NN; ++n) {
          const long va = *reinterpret_cast<const long*>(&s_v[vpg][16 * n + lr][vpage_off]);
          const v4i c = __builtin_amdgcn_mfma_i32_16x16x32_i8(va, wb, v4i{0, 0, 0, 0}, 0, 0, 0);
#pragma unroll
          for (int i = 0; i < 4; ++i) O[n][i] += swg[g] * (float)c[i];
        }
      }
    } else {
      const long wb0 = (long)(((uint64_t)wpk[0][1] << 32) | wpk[0][0]);
      const long wb1 = (long)(((uint64_t)wpk[1][1] << 32) | wpk[1][0]);
#pragma unroll
      for (int n = 0; n < NN; ++n) {
        const long va0 = *reinterpret_cast<const long*>(&s_v[lg >> 1][16 * n + lr][vpage_off]);
        const long va1 = *reinterpret_cast<const long*>(&s_v[2 + (lg >> 1)][16 * n + lr][vpage_off]);
        v4i c = __builtin_amdgcn_mfma_i32_16x16x32_i8(va0, wb0, v4i{0, 0, 0, 0}, 0, 0, 0);
        c = __builtin_amdgcn_mfma_i32_16x16x32_i8(va1, wb1, c, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) O[n][i] += swg[0] * (float)c[i];
      }
    }
  }

  // ---- O / l and store: lane l holds row l%16, dims 16n + 4(l/16) + i ----------
  const float l_row = row_sum4(lsum);
  if (!row_ok) return;
  const float inv = 1.0f / l_row;
  float* dst = a.out + qrow * D + 4 * lg;
#pragma unroll
  for (int n = 0; n < NN; ++n)
    *reinterpret_cast<float4*>(dst + 16 * n) =
        make_float4(O[n][0] * inv, O[n][1] * inv, O[n][2] * inv, O[n][3] * inv);
}

hipError_t launch_prefix_prefill(const PrefillArgs& a, hipStream_t stream) {
  if (a.num_seqs == 0 || a.max_query_len == 0) return hipSuccess;
  const int64_t rows = (int64_t)a.max_query_len * a.group;
  const int64_t tiles = (rows + kRows - 1) / kRows;
  dim3 grid((unsigned)tiles, (unsigned)a.num_kv_heads, (unsigned)a.num_seqs);
  dim3 block(kNW * kWave);
#define I8KV_PREFILL_CASE(DD, GG)                                                     \
  if (a.head_dim == DD && a.w_group == GG) {                                          \
    hipLaunchKernelGGL((prefix_prefill_kernel<DD, GG>), grid, block, 0, stream, a);   \
    return hipGetLastError();                                                         \
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
