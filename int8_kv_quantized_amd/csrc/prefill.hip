// Chunked prefill with history over the INT8 KV cache: one online softmax
// over the history pages and the causal chunk.
//
// What is computed follows the page "Implementing INT8 PV MMAC on a gfx936
// DCU: V-scale fusion, probability quantization, fragment grouping":
//   section 2   score = acc * sQ * sK / sqrt(d);
//   section 2.1 state (m, l, o): m' = max(m, max s), alpha = exp(m - m'),
//               p~ = exp(s - m'), W = p~ * sV quantized per G-key group,
//               o = alpha o + sum sW (Wq x Vq), l = alpha l + sum p~, O = o / l;
//   section 3/4 W is operand A, V operand B, one scale per group of exactly
//               the keys one MFMA chain consumes;
// and "INT8 KV and INT8 MMAC attention inference optimisation on a gfx936
// DCU", section 3.2 (history and chunk in the same online softmax) and
// section 4.2 (more query rows per workgroup so each K/V tile is reused).
//
// gfx950 mapping.  A workgroup of 4 waves owns 128 consecutive flattened rows
// (query token, q head of the GQA group) of one (sequence, KV head); wave w
// owns rows 32w..32w+31, lane l (and its partner l^32) row l%32.  Per 64-key
// tile, K and V pages are staged in LDS in their cache layouts.
//  * QK is computed transposed, S^T = K Q^T, with v_mfma_i32_32x32x32_i8:
//    operand A = 32 keys (16 head-dim bytes per lane from LDS), operand B =
//    the int8 queries (held in registers for the whole loop).  The A rows are
//    a permutation of the keys chosen so that output register v of lane l is
//    key 16*(l/32) + v: each lane holds 16 consecutive keys of its row.
//  * Those 16 keys are exactly the operand-A slice of the PV MFMA
//    (v_mfma_i32_32x32x32_i8, K = 32 keys): W is quantized and packed in
//    registers and never leaves them.  Operand B is V straight from the LDS
//    copy of the page (16 tokens of one dim are 16 contiguous bytes).
//  * G = 32: one PV MFMA per 32-key group and 32 output dims, rescaled by the
//    group's sW.  G = 64: two MFMAs chained in int32 (same scale), one rescale.
#include "device_common.hpp"
#include "kernels.hpp"

namespace i8kv {

namespace {

constexpr int kNW = 4;         // waves per workgroup
constexpr int kRows = 32 * kNW;  // flattened rows per workgroup
constexpr int kKT = 64;        // keys per tile

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// A-row r of the transposed QK reads key perm(r) so that output register v
// of lane l holds key 16*(l/32) + v.
__device__ __forceinline__ int key_of_arow(int r) {
  const int j = r >> 3, h = (r >> 2) & 1, i = r & 3;
  return 16 * h + 4 * j + i;
}

}  // namespace

template <int D, int G>
__global__ __launch_bounds__(256) void prefix_prefill_kernel(PrefillArgs a) {
  constexpr int NC = D / 32;  // 32-dim k-steps (QK) and 32-dim output tiles (PV)
  __shared__ __attribute__((aligned(16))) int8_t s_k[D / 16][kKT][16];
  __shared__ __attribute__((aligned(16))) int8_t s_v[kKT / 16][D][16];
  __shared__ float s_sk[kKT], s_sv[kKT];
  __shared__ __attribute__((aligned(16))) float s_row[kNW][32];
  __shared__ int s_pid[kKT / 16];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int hl = lane >> 5, rl = lane & 31;
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
  const int fr = row0 + 32 * w + rl;
  const bool row_ok = fr < nrows_seq;
  const int tok = row_ok ? fr / grp : 0;
  const int head = row_ok ? fr % grp : 0;
  const int pos = ctx + tok;
  const size_t qrow = (size_t)(q0 + tok) * a.num_q_heads + (size_t)kv * grp + head;

  v4i qb[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c)
    qb[c] = row_ok ? *reinterpret_cast<const v4i*>(a.q_int8 + qrow * D + 32 * c + 16 * hl)
                   : v4i{0, 0, 0, 0};
  const float sq = row_ok ? a.q_scale[qrow] : 0.0f;

  const int last_fr = min(row0 + kRows, nrows_seq) - 1;
  const int nkeys = ctx + last_fr / grp + 1;  // keys visible to the workgroup's last row
  const int wave_last_fr = min(row0 + 32 * w + 31, nrows_seq - 1);
  const int wave_nkeys = (wave_last_fr >= row0 + 32 * w) ? ctx + wave_last_fr / grp + 1 : 0;
  const int ntiles = (nkeys + kKT - 1) / kKT;
  const int npages_seq = min((seq_len + kBlockSize - 1) / kBlockSize, a.max_blocks_per_seq);

  float m = -INFINITY;
  float lpart = 0.0f;
  float O[NC][16];
#pragma unroll
  for (int n = 0; n < NC; ++n)
#pragma unroll
    for (int v = 0; v < 16; ++v) O[n][v] = 0.0f;

  const int arow_key = key_of_arow(rl);

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
    // K: 4 pages x D/16 chunks x 16 keys, 16 bytes each
    for (int u = tid; u < 4 * D; u += blockDim.x) {
      const int i = u / D, rem = u % D, ch = rem / 16, key = rem % 16;
      const int pid = s_pid[i];
      v4i val = {0, 0, 0, 0};
      if (pid >= 0)
        val = *reinterpret_cast<const v4i*>(
            a.k_cache + (((size_t)pid * Hkv + kv) * (D / 16) + ch) * 256 + key * 16);
      *reinterpret_cast<v4i*>(&s_k[ch][16 * i + key][0]) = val;
    }
    // V: 4 pages x D dims, 16 tokens each
    for (int u = tid; u < 4 * D; u += blockDim.x) {
      const int i = u / D, d = u % D;
      const int pid = s_pid[i];
      v4i val = {0, 0, 0, 0};
      if (pid >= 0)
        val = *reinterpret_cast<const v4i*>(a.v_cache + (((size_t)pid * Hkv + kv) * D + d) * 16);
      *reinterpret_cast<v4i*>(&s_v[i][d][0]) = val;
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
    if (k0 >= wave_nkeys) continue;  // this wave's rows see no key of the tile

    // ---- S^T = K Q^T for the two 32-key halves --------------------------
    float sc[2][16];
    float mt = -INFINITY;
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      v16i acc = {};
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const v4i ka = *reinterpret_cast<const v4i*>(&s_k[2 * c + hl][32 * kh + arow_key][0]);
        acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(ka, qb[c], acc, 0, 0, 0);
      }
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int kl = 32 * kh + 16 * hl + v;
        const int key = k0 + kl;
        float x = (float)acc[v] * sq;
        x = x * s_sk[kl];
        x = x * a.softmax_scale;
        x = (row_ok && key <= pos) ? x : -INFINITY;
        sc[kh][v] = x;
        mt = fmaxf(mt, x);
      }
    }
    mt = fmaxf(mt, __shfl_xor(mt, 32, kWave));
    const float m_new = fmaxf(m, mt);
    const float alpha = (m_new == -INFINITY) ? 1.0f : expf(m - m_new);
    m = m_new;

    // ---- p~, l, W and its group quantization -----------------------------
    v4i wq[2];
    float swh[2];
    float psum = 0.0f;
    float Wt[2][16];
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float pt = (sc[kh][v] == -INFINITY) ? 0.0f : expf(sc[kh][v] - m_new);
        psum += pt;
        Wt[kh][v] = pt * s_sv[32 * kh + 16 * hl + v];
      }
    lpart = alpha * lpart + psum;
    float am[2];
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      float x = 0.0f;
#pragma unroll
      for (int v = 0; v < 16; ++v) x = fmaxf(x, Wt[kh][v]);
      am[kh] = fmaxf(x, __shfl_xor(x, 32, kWave));
    }
    if constexpr (G == 64) am[0] = am[1] = fmaxf(am[0], am[1]);
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      const float sw = am[kh] > 0.0f ? am[kh] / 127.0f : 0.0f;
      swh[kh] = sw;
      uint32_t pk[4] = {0, 0, 0, 0};
      if (am[kh] > 0.0f) {
#pragma unroll
        for (int v = 0; v < 16; ++v)
          pk[v / 4] |= (uint32_t)(quantize_code(Wt[kh][v], sw) & 0xff) << (8 * (v % 4));
      }
      wq[kh] = v4i{(int)pk[0], (int)pk[1], (int)pk[2], (int)pk[3]};
    }

    // ---- rescale O by alpha of each output row -------------------------------
    // PV output register v of lane l holds row 8*(v/4) + 4*(l/32) + v%4.
    if (hl == 0) s_row[w][rl] = alpha;
    wave_lds_sync();
    float arow[16];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float4 q4 = *reinterpret_cast<const float4*>(&s_row[w][8 * j + 4 * hl]);
      arow[4 * j + 0] = q4.x;
      arow[4 * j + 1] = q4.y;
      arow[4 * j + 2] = q4.z;
      arow[4 * j + 3] = q4.w;
    }
    wave_lds_sync();
#pragma unroll
    for (int n = 0; n < NC; ++n)
#pragma unroll
      for (int v = 0; v < 16; ++v) O[n][v] *= arow[v];

    // ---- PV: int8 MFMA per group, rescaled by sW of each row ----------------
    constexpr int NG = (G == 32) ? 2 : 1;
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      if (hl == 0) s_row[w][rl] = swh[g];
      wave_lds_sync();
      float srow[16];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float4 q4 = *reinterpret_cast<const float4*>(&s_row[w][8 * j + 4 * hl]);
        srow[4 * j + 0] = q4.x;
        srow[4 * j + 1] = q4.y;
        srow[4 * j + 2] = q4.z;
        srow[4 * j + 3] = q4.w;
      }
      wave_lds_sync();
#pragma unroll
      for (int n = 0; n < NC; ++n) {
        v16i acc = {};
        if constexpr (G == 32) {
          const v4i vb = *reinterpret_cast<const v4i*>(&s_v[2 * g + hl][32 * n + rl][0]);
          acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(wq[g], vb, acc, 0, 0, 0);
        } else {
#pragma unroll
          for (int kh = 0; kh < 2; ++kh) {
            const v4i vb = *reinterpret_cast<const v4i*>(&s_v[2 * kh + hl][32 * n + rl][0]);
            acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(wq[kh], vb, acc, 0, 0, 0);
          }
        }
#pragma unroll
        for (int v = 0; v < 16; ++v) O[n][v] += srow[v] * (float)acc[v];
      }
    }
  }

  // ---- O / l and store --------------------------------------------------------
  const float l_row = lpart + __shfl_xor(lpart, 32, kWave);
  if (hl == 0) s_row[w][rl] = l_row;
  wave_lds_sync();
  float lrow[16];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float4 q4 = *reinterpret_cast<const float4*>(&s_row[w][8 * j + 4 * hl]);
    lrow[4 * j + 0] = q4.x;
    lrow[4 * j + 1] = q4.y;
    lrow[4 * j + 2] = q4.z;
    lrow[4 * j + 3] = q4.w;
  }
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int r = 8 * (v / 4) + 4 * hl + (v % 4);
    const int fr2 = row0 + 32 * w + r;
    if (fr2 >= nrows_seq) continue;
    const int tk = fr2 / grp, hd = fr2 % grp;
    float* dst = a.out + ((size_t)(q0 + tk) * a.num_q_heads + (size_t)kv * grp + hd) * D;
    const float inv = 1.0f / lrow[v];
#pragma unroll
    for (int n = 0; n < NC; ++n) dst[32 * n + rl] = O[n][v] * inv;
  }
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
