// Paged decode over the INT8 KV cache, one query per sequence.
//
// What is computed follows the page "Implementing INT8 PV MMAC on a gfx936
// DCU: V-scale fusion, probability quantization, fragment grouping":
//   section 2  score_i = acc_i * sQ * sK_i / sqrt(d) from the int32 QK sum;
//   section 2.2 256-token partitions, each with its own max m_p and sum l_p,
//              P_i = exp(score_i - m_p) / l_p and W_i = P_i * sV_i, outputs
//              merged across partitions with log-sum-exp weights;
//   section 1  per group of G tokens sW = max W / 127, Wq = round(W / sW),
//              O_group = (Wq x Vq) * sW with an int8 product;
//   section 3  W is operand A (rows = query heads), V is operand B;
//   section 4  each scale is computed on exactly the tokens its matrix
//              instruction consumes.
// and the page "INT8 KV and INT8 MMAC attention inference optimisation on a
// gfx936 DCU", section 3.3 (read the paged int8 K/V directly; no bf16 copy).
//
// gfx950 mapping (one workgroup = 4 waves = one 256-token partition of one
// (sequence, KV head)):
//  * QK: v_mfma_i32_16x16x64_i8 with A = the GQA group's int8 queries (rows =
//    q heads, zero-padded to 16) and B = one 16-token page: lane l loads the
//    16 head-dim bytes of token l%16, chunk 4c + l/16 -- one 16-byte load per
//    lane, 1 KiB contiguous per wave instruction.  Wave w owns pages 4w..4w+3.
//  * Softmax: per-head max / sum over the 16 lanes of a row, then across
//    waves through LDS.  The elementwise chain is the fp32 one the pages use
//    (IEEE divide, correctly rounded exp, fp64 sum rounded to fp32), so Wq is
//    decided exactly as the definition does.
//  * PV: v_mfma_i32_16x16x64_i8 with A = Wq read back from an LDS tile
//    (rows = heads, 16 tokens per lane) and B = 16 tokens of one V row
//    (V [page, h, d, 16] has the 16 tokens of a page contiguous per dim):
//    each 64-token MFMA consumes pages 4g..4g+3, lane group j holding page
//    4g + j.  G = 64 is one MFMA per group; for G = 32 operand A is masked to
//    lane groups {0,1} resp. {2,3}, so each MFMA consumes exactly one group.
//    Wave w owns dims [w*D/4, (w+1)*D/4) for all 256 tokens.
//  * Merge: partials (m, l, o) go to the workspace; the last workgroup to
//    finish a node of `fanout` partitions merges them (fence + atomic
//    counter), and the last node merges the nodes into the output.
#include "device_common.hpp"
#include "kernels.hpp"

namespace i8kv {

namespace {
constexpr int kMaxMergeChildren = 64;
constexpr int kWqStride = 256 + 16;  // LDS row pitch of the Wq tile (bytes)

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
}  // namespace

DecodePlan make_decode_plan(int32_t num_seqs, int32_t num_kv_heads, int32_t group,
                            int32_t head_dim, int32_t max_seq_len) {
  DecodePlan p{};
  p.num_seqs = num_seqs;
  p.num_kv_heads = num_kv_heads;
  p.group = group;
  p.head_dim = head_dim;
  p.max_parts = max_seq_len > 0 ? (max_seq_len + kPartition - 1) / kPartition : 1;
  int f = 2;
  while (f * f < p.max_parts) ++f;
  p.fanout = f;
  p.max_nodes = (p.max_parts + f - 1) / f;
  const size_t units = (size_t)num_seqs * num_kv_heads;
  size_t off = 0;
  p.off_part_o = off;
  off = align_up(off + units * p.max_parts * group * head_dim * sizeof(float), 256);
  p.off_part_ml = off;
  off = align_up(off + units * p.max_parts * group * 2 * sizeof(float), 256);
  p.off_node_o = off;
  off = align_up(off + units * p.max_nodes * group * head_dim * sizeof(float), 256);
  p.off_node_ml = off;
  off = align_up(off + units * p.max_nodes * group * 2 * sizeof(float), 256);
  p.off_cnt1 = off;
  off = align_up(off + units * p.max_nodes * sizeof(int32_t), 256);
  p.off_cnt2 = off;
  off = align_up(off + units * sizeof(int32_t), 256);
  p.bytes = off;
  return p;
}

// Merge n partial states (m, l, o) of the grp heads of one (seq, KV head):
//   M = max m_c, w_c = l_c exp(m_c - M), o = sum w_c o_c / sum w_c.
// Writes o to dst_o [grp, D] and, if dst_ml is given, (M, sum w_c) per head.
template <int D>
__device__ void merge_children(const float* __restrict__ src_o, const float* __restrict__ src_ml,
                               int n, int grp, float* __restrict__ dst_o,
                               float* __restrict__ dst_ml, float (*s_w)[kMaxMergeChildren]) {
  const int tid = threadIdx.x;
  if (tid < grp) {
    const int h = tid;
    float M = -INFINITY;
    for (int c = 0; c < n; ++c) M = fmaxf(M, src_ml[((size_t)c * grp + h) * 2]);
    float wsum = 0.0f;
    for (int c = 0; c < n; ++c) {
      const float m = src_ml[((size_t)c * grp + h) * 2];
      const float l = src_ml[((size_t)c * grp + h) * 2 + 1];
      const float w = l * expf(m - M);
      s_w[h][c] = w;
      wsum += w;
    }
    const float inv = 1.0f / wsum;
    for (int c = 0; c < n; ++c) s_w[h][c] *= inv;
    if (dst_ml) {
      dst_ml[h * 2] = M;
      dst_ml[h * 2 + 1] = wsum;
    }
  }
  __syncthreads();
  const int total4 = grp * D / 4;
  for (int i = tid; i < total4; i += blockDim.x) {
    const int h = (i * 4) / D;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int c = 0; c < n; ++c) {
      const float4 v = reinterpret_cast<const float4*>(src_o + (size_t)c * grp * D)[i];
      const float w = s_w[h][c];
      acc.x += w * v.x;
      acc.y += w * v.y;
      acc.z += w * v.z;
      acc.w += w * v.w;
    }
    reinterpret_cast<float4*>(dst_o)[i] = acc;
  }
}

template <int D, int G>
__global__ __launch_bounds__(256) void paged_decode_kernel(DecodeArgs a) {
  constexpr int NC = D / 64;    // 64-byte k-steps of the QK product
  constexpr int DW = D / 4;     // output dims per wave
  constexpr int NCW = DW / 16;  // 16-dim output tiles per wave
  constexpr int NGW = 64 / G;   // W groups per 64-token MFMA (1 or 2)

  __shared__ __attribute__((aligned(16))) uint8_t s_wq[16 * kWqStride];
  __shared__ float s_sw[16][kPartition / G];
  __shared__ float s_red_m[4][16];
  __shared__ double s_red_l[4][16];
  __shared__ float s_w[16][kMaxMergeChildren];
  __shared__ int s_flag;

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int lg = lane >> 4, lr = lane & 15;
  const int p = blockIdx.x, kv = blockIdx.y, s = blockIdx.z;
  const int grp = a.group;
  const int Hkv = a.num_kv_heads;

  int L = a.seq_lens[s];
  L = min(max(L, 0), a.max_seq_len);
  const int P_s = (L + kPartition - 1) / kPartition;
  float* out_base = a.out + ((size_t)s * a.num_q_heads + (size_t)kv * grp) * D;
  if (L == 0) {
    if (p == 0)
      for (int i = tid; i < grp * D; i += blockDim.x) out_base[i] = 0.0f;
    return;
  }
  if (p >= P_s) return;

  const int tok0 = p * kPartition;
  const int npages = min(16, (L + kBlockSize - 1) / kBlockSize - p * 16);

  // ---- page ids of this partition (lane j < 16 holds page j) -------------
  int my_pid = 0;
  if (lane < npages) {
    my_pid = a.block_tables[(size_t)s * a.max_blocks_per_seq + p * 16 + lane];
    my_pid = min(max(my_pid, 0), a.num_blocks - 1);
  }

  // ---- operand loads: Q (A), own K pages (B), V rows for own dims (B) ----
  v4i qa[NC];
  {
    const bool vh = lr < grp;
    const int8_t* qp = a.q_int8 +
                       ((size_t)s * a.num_q_heads + (size_t)kv * grp + (vh ? lr : 0)) * D + 16 * lg;
#pragma unroll
    for (int c = 0; c < NC; ++c)
      qa[c] = vh ? *reinterpret_cast<const v4i*>(qp + 64 * c) : v4i{0, 0, 0, 0};
  }
  v4i kb[4][NC];
  int pidw[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int pi = 4 * w + j;
    pidw[j] = __shfl(my_pid, pi & 15, kWave);
    const int8_t* base = a.k_cache + ((size_t)pidw[j] * Hkv + kv) * (size_t)(D / 16) * 256;
#pragma unroll
    for (int c = 0; c < NC; ++c)
      kb[j][c] = (pi < npages) ? *reinterpret_cast<const v4i*>(base + (4 * c + lg) * 256 + lr * 16)
                               : v4i{0, 0, 0, 0};
  }
  v4i vb[4][NCW];
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int pi = 4 * g + lg;  // page of this lane group in 64-token group g
    const int pid = __shfl(my_pid, pi, kWave);
    const int8_t* base = a.v_cache + ((size_t)pid * Hkv + kv) * (size_t)D * 16;
#pragma unroll
    for (int c = 0; c < NCW; ++c) {
      const int d = w * DW + 16 * c + lr;
      vb[g][c] = (pi < npages) ? *reinterpret_cast<const v4i*>(base + d * 16) : v4i{0, 0, 0, 0};
    }
  }
  float sk[4], sv[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int tok = tok0 + 64 * w + 16 * j + lr;
    const bool ok = tok < L;
    const size_t idx = ((size_t)pidw[j] * kBlockSize + lr) * Hkv + kv;
    sk[j] = ok ? a.k_scale[idx] : 0.0f;
    sv[j] = ok ? a.v_scale[idx] : 0.0f;
  }
  float sq[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int h = 4 * lg + r;
    sq[r] = h < grp ? a.q_scale[(size_t)s * a.num_q_heads + (size_t)kv * grp + h] : 0.0f;
  }

  // ---- QK and score recovery ---------------------------------------------
  float sc[4][4];  // [page j][head r]: token tok0 + 64w + 16j + lr, head 4lg + r
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    v4i acc = {0, 0, 0, 0};
#pragma unroll
    for (int c = 0; c < NC; ++c)
      acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(qa[c], kb[j][c], acc, 0, 0, 0);
    const int tok = tok0 + 64 * w + 16 * j + lr;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float x = (float)acc[r] * sq[r];
      x = x * sk[j];
      x = x * a.softmax_scale;
      sc[j][r] = (tok < L && 4 * lg + r < grp) ? x : -INFINITY;
    }
  }

  // ---- partition softmax: max, exp, fp64 sum --------------------------------
  float M[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float m = fmaxf(fmaxf(sc[0][r], sc[1][r]), fmaxf(sc[2][r], sc[3][r]));
    m = group_max<16>(m);
    if (lr == 0) s_red_m[w][4 * lg + r] = m;
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int h = 4 * lg + r;
    M[r] = fmaxf(fmaxf(s_red_m[0][h], s_red_m[1][h]), fmaxf(s_red_m[2][h], s_red_m[3][h]));
  }
  float e[4][4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    double ls = 0.0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      e[j][r] = (sc[j][r] == -INFINITY) ? 0.0f : exp_f32_rn(sc[j][r] - M[r]);
      ls += (double)e[j][r];
    }
    ls = group_sum<16>(ls);
    if (lr == 0) s_red_l[w][4 * lg + r] = ls;
  }
  __syncthreads();
  float lf[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int h = 4 * lg + r;
    lf[r] = (float)(s_red_l[0][h] + s_red_l[1][h] + s_red_l[2][h] + s_red_l[3][h]);
  }

  // ---- W = P * sV and group quantization ------------------------------------
  float W[4][4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float P = (e[j][r] != 0.0f) ? e[j][r] / lf[r] : 0.0f;
      W[j][r] = P * sv[j];
    }
#pragma unroll
  for (int gg = 0; gg < NGW; ++gg) {
    constexpr int JP = 4 / NGW;  // pages per group within the wave
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float am = 0.0f;
#pragma unroll
      for (int jj = 0; jj < JP; ++jj) am = fmaxf(am, W[gg * JP + jj][r]);
      am = group_max<16>(am);
      const float sw = am > 0.0f ? am / 127.0f : 0.0f;
      const int h = 4 * lg + r;
#pragma unroll
      for (int jj = 0; jj < JP; ++jj) {
        const int j = gg * JP + jj;
        const int q = am > 0.0f ? quantize_code(W[j][r], sw) : 0;
        s_wq[h * kWqStride + 64 * w + 16 * j + lr] = (uint8_t)q;
      }
      if (lr == 0) s_sw[h][w * NGW + gg] = sw;
    }
  }
  __syncthreads();

  // ---- PV: int8 MFMA per group, rescaled by sW into fp32 ---------------------
  float o[NCW][4];
#pragma unroll
  for (int c = 0; c < NCW; ++c)
#pragma unroll
    for (int r = 0; r < 4; ++r) o[c][r] = 0.0f;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const v4i wa = *reinterpret_cast<const v4i*>(&s_wq[lr * kWqStride + 64 * g + 16 * lg]);
    if constexpr (G == 64) {
      float swr[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) swr[r] = s_sw[4 * lg + r][g];
#pragma unroll
      for (int c = 0; c < NCW; ++c) {
        const v4i acc =
            __builtin_amdgcn_mfma_i32_16x16x64_i8(wa, vb[g][c], v4i{0, 0, 0, 0}, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) o[c][r] += swr[r] * (float)acc[r];
      }
    } else {
      const v4i zero = {0, 0, 0, 0};
      const v4i wlo = lg < 2 ? wa : zero;
      const v4i whi = lg < 2 ? zero : wa;
      float slo[4], shi[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        slo[r] = s_sw[4 * lg + r][2 * g];
        shi[r] = s_sw[4 * lg + r][2 * g + 1];
      }
#pragma unroll
      for (int c = 0; c < NCW; ++c) {
        const v4i alo = __builtin_amdgcn_mfma_i32_16x16x64_i8(wlo, vb[g][c], zero, 0, 0, 0);
        const v4i ahi = __builtin_amdgcn_mfma_i32_16x16x64_i8(whi, vb[g][c], zero, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          o[c][r] += slo[r] * (float)alo[r];
          o[c][r] += shi[r] * (float)ahi[r];
        }
      }
    }
  }

  // ---- single partition: write the output directly ---------------------------
  if (P_s == 1) {
#pragma unroll
    for (int c = 0; c < NCW; ++c)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int h = 4 * lg + r;
        if (h < grp) out_base[(size_t)h * D + w * DW + 16 * c + lr] = o[c][r];
      }
    return;
  }

  // ---- write the partition partial and merge -------------------------------
  const size_t unit = (size_t)s * Hkv + kv;
  float* po = a.part_o + ((unit * a.max_parts + p) * grp) * D;
#pragma unroll
  for (int c = 0; c < NCW; ++c)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = 4 * lg + r;
      if (h < grp) po[(size_t)h * D + w * DW + 16 * c + lr] = o[c][r];
    }
  if (w == 0 && lr == 0) {
    float* pml = a.part_ml + ((unit * a.max_parts + p) * grp) * 2;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = 4 * lg + r;
      if (h < grp) {
        pml[h * 2] = M[r];
        pml[h * 2 + 1] = lf[r];
      }
    }
  }
  __threadfence();
  __syncthreads();

  const int F = a.fanout;
  const int node = p / F;
  const int n1 = min(F, P_s - node * F);
  const int nnodes = (P_s + F - 1) / F;
  if (tid == 0) {
    int* c = a.cnt1 + unit * a.max_nodes + node;
    const int old = atomicAdd(c, 1);
    const int last = (old == n1 - 1);
    if (last) atomicExch(c, 0);
    s_flag = last;
  }
  __syncthreads();
  if (!s_flag) return;
  __threadfence();
  {
    const float* so = a.part_o + ((unit * a.max_parts + (size_t)node * F) * grp) * D;
    const float* sm = a.part_ml + ((unit * a.max_parts + (size_t)node * F) * grp) * 2;
    if (nnodes == 1) {
      merge_children<D>(so, sm, n1, grp, out_base, nullptr, s_w);
      return;
    }
    merge_children<D>(so, sm, n1, grp, a.node_o + ((unit * a.max_nodes + node) * grp) * D,
                      a.node_ml + ((unit * a.max_nodes + node) * grp) * 2, s_w);
  }
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    int* c = a.cnt2 + unit;
    const int old = atomicAdd(c, 1);
    const int last = (old == nnodes - 1);
    if (last) atomicExch(c, 0);
    s_flag = last;
  }
  __syncthreads();
  if (!s_flag) return;
  __threadfence();
  merge_children<D>(a.node_o + (unit * a.max_nodes * grp) * D,
                    a.node_ml + (unit * a.max_nodes * grp) * 2, nnodes, grp, out_base, nullptr,
                    s_w);
}

hipError_t launch_paged_decode(const DecodeArgs& a, hipStream_t stream) {
  if (a.num_seqs == 0) return hipSuccess;
  dim3 grid((unsigned)a.max_parts, (unsigned)a.num_kv_heads, (unsigned)a.num_seqs);
  dim3 block(256);
#define I8KV_DECODE_CASE(DD, GG)                                                        \
  if (a.head_dim == DD && a.w_group == GG) {                                            \
    hipLaunchKernelGGL((paged_decode_kernel<DD, GG>), grid, block, 0, stream, a);       \
    return hipGetLastError();                                                           \
  }
  I8KV_DECODE_CASE(64, 32)
  I8KV_DECODE_CASE(64, 64)
  I8KV_DECODE_CASE(128, 32)
  I8KV_DECODE_CASE(128, 64)
  I8KV_DECODE_CASE(256, 32)
  I8KV_DECODE_CASE(256, 64)
#undef I8KV_DECODE_CASE
  return hipErrorInvalidValue;
}

}  // namespace i8kv
