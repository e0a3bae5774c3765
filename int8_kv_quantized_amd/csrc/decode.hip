// Paged decode over the INT8 KV cache, one query per sequence.
//
// What is computed follows the page "Implementing INT8 PV MMAC on a gfx936
// DCU: V-scale fusion, probability quantization, fragment grouping":
//   section 2   score_i = acc_i * sQ * sK_i / sqrt(d) from the int32 QK sum;
//   section 2.2 256-token partitions, each with its own max m_p and sum l_p,
//               P_i = exp(score_i - m_p) / l_p and W_i = P_i * sV_i; partition
//               outputs merged with log-sum-exp weights;
//   section 1   per group of G tokens sW = max W / 127, Wq = round(W / sW),
//               O_group = (Wq x Vq) * sW with an int8 product;
//   section 3   W is operand A (rows = query heads), V is operand B;
//   section 4   each scale covers exactly the tokens its MFMA consumes;
// and the page "INT8 KV and INT8 MMAC attention inference optimisation on a
// gfx936 DCU", section 3.3 (the paged int8 K/V are read directly).
//
// Two kernels, no cross-workgroup synchronization:
//
// 1. paged_decode_partition_kernel: one workgroup of 8 waves (4 for D <= 128)
//    per (256-token partition, KV head, sequence).  Two load round trips:
//    (1) sequence length, block-table entries, queries and their scales;
//    (2) all scales and K bytes of the partition (16-byte loads), then each
//    wave's V bytes as soon as its QK has consumed K (~128 KiB per workgroup
//    in flight).  Then:
//    * QK: v_mfma_i32_16x16x64_i8, A = the GQA group's int8 queries (rows =
//      q heads, zero-padded to 16), B = one page: lane l holds the 16
//      head-dim bytes of token l%16 in chunk 4c + l/16.  Wave w owns pages
//      2w, 2w+1 (4w..4w+3 for D <= 128).  Scores of the real heads go to LDS.
//    * Softmax and W quantization: wave h owns head h, lane l tokens
//      4l..4l+3, so max and sum are one-wave reductions and no lane works on
//      padding rows.  The chain is the definition's fp32 one (fp32 exp rounded
//      once from fp64, fp64 sum rounded to fp32, IEEE divides), so Wq is
//      decided as the definition decides it.
//    * PV: v_mfma_i32_16x16x64_i8, A = Wq from LDS (rows = heads, 16 tokens
//      per lane), B = 16 tokens of one V row (one page, one dim: 16 contiguous
//      bytes); the MFMA over 64 tokens consumes pages 4g..4g+3, lane group j
//      page 4g+j.  G = 64: one MFMA per group; G = 32: operand A is masked to
//      lane groups {0,1} resp. {2,3} so each MFMA consumes exactly one group.
//      Wave w owns output dims [w D/NW, (w+1) D/NW) of the NW waves.
//    A single-partition sequence writes the output; otherwise (m_p, l_p, o_p)
//    go to the workspace.
// 2. paged_decode_merge_kernel: one wave per (q head, sequence, 32 output
//    dims) merges the partitions, O = sum w_p o_p / sum w_p with
//    w_p = l_p exp(m_p - M).
// The two kernels also run alone (DecodeArgs::stage): the partitions with
// every sequence's partials written to the workspace, or the merge of a
// workspace so filled -- the split a decode sharded over the partitions of a
// sequence needs (partials computed where the pages are, merged once).
#include "device_common.hpp"
#include "kernels.hpp"

namespace i8kv {

namespace {
size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
constexpr int kTokStride = kPartition + 4;  // LDS pitch of the score tile (floats)
constexpr int kWqStride = kPartition + 16;  // LDS pitch of the Wq tile (bytes)
constexpr int kWbStride = kPartition + 8;   // LDS pitch of the bf16 W tile (elements)

}  // namespace

DecodePlan make_decode_plan(int32_t num_seqs, int32_t num_kv_heads, int32_t group,
                            int32_t head_dim, int32_t max_seq_len) {
  DecodePlan p{};
  p.num_seqs = num_seqs;
  p.num_kv_heads = num_kv_heads;
  p.group = group;
  p.head_dim = head_dim;
  p.max_parts = max_seq_len > 0 ? (max_seq_len + kPartition - 1) / kPartition : 1;
  const size_t units = (size_t)num_seqs * num_kv_heads * p.max_parts * group;
  p.off_part_o = 0;
  p.off_part_ml = align_up(units * head_dim * sizeof(float), 256);
  p.bytes = align_up(p.off_part_ml + units * 2 * sizeof(float), 256);
  return p;
}

// Waves per partition workgroup and the work of each.
template <int D>
struct DecodeShape {
  static constexpr int NW = D >= 256 ? 8 : 4;  // waves (4 for D <= 128: more workgroups per CU)
  static constexpr int PPW = 16 / NW;          // pages per wave in QK
  static constexpr int DW = D / NW;            // output dims per wave in PV
  static constexpr int NCW = DW / 16;          // 16-dim PV tiles per wave
};

// PV variants: the method's int8 W groups, the BF16-PV ablation (W = P*sV in
// bf16), and UINT8 W groups (codes 0..255 against max W / 255).
enum : int { kPvInt8 = 0, kPvBf16 = 1, kPvUint8 = 2 };

// Minimum waves per SIMD the compiler must allow: 4 for the int8-PV D = 128
// kernels that fit 128 VGPRs without spilling, so four 4-wave workgroups share
// a CU (the many-workgroup MHA decode measured 126 -> 122 us); the others keep
// what their registers give (the UINT8-W and ablation variants, and the
// several-query G = 32 variant, would spill under the cap).
template <int D, int G, int PVM, bool MQ, bool QB>
constexpr int decode_min_waves() {
  return (D == 128 && PVM == kPvInt8 && !QB && !(MQ && G == 32)) ? 4 : 1;
}

// QB: the BF16-QK ablation -- the bf16 queries (not quantized) against the
// int8 K codes taken exactly as bf16, v_mfma_f32_16x16x32_bf16 with fp32
// accumulation, score = (dot * sK) * softmax_scale; the rest is unchanged.
// Grid modes, chosen at launch: one round of workgroups (at most one per CU);
// several rounds -- the length is checked before any vector load, so a
// workgroup past its sequence leaves without waiting for loads it would not
// use; several rounds with kilobytes of partials per workgroup -- also the
// partials go out with non-temporal stores.
enum : int { kOneRound = 0, kRounds = 1, kRoundsNt = 2 };

template <int D, int G, bool FUSED, int PVM, bool MQ, bool QB, int MODE = kOneRound>
__global__ __launch_bounds__(DecodeShape<D>::NW * kWave, (decode_min_waves<D, G, PVM, MQ, QB>())) void
paged_decode_partition_kernel(
    DecodeArgs a) {
  constexpr bool BPV = PVM == kPvBf16;
  constexpr bool U8W = PVM == kPvUint8;
  constexpr int NW = DecodeShape<D>::NW;
  constexpr int NT = NW * kWave;
  constexpr int PPW = DecodeShape<D>::PPW;
  constexpr int NCW = DecodeShape<D>::NCW;
  constexpr int NC = D / 64;          // 64-byte k-steps of the QK product
  constexpr int NGP = kPartition / G; // W groups per partition

  __shared__ __attribute__((aligned(16))) float s_sc[16 * kTokStride];
  __shared__ __attribute__((aligned(16))) uint8_t s_wq[16 * kWqStride];
  __shared__ __attribute__((aligned(16))) float s_sv[kPartition];
  __shared__ float s_sw[16][NGP];
  __shared__ float s_M[16], s_L[16];
  // fused step: the group's quantized queries and the newest token's K/V codes
  __shared__ __attribute__((aligned(16))) int8_t s_q[FUSED ? 16 : 1][FUSED ? D : 16];
  __shared__ __attribute__((aligned(16))) int8_t s_nk[FUSED ? D : 16], s_nv[FUSED ? D : 16];
  __shared__ float s_qs[16], s_nsc[2];
  // BF16-PV ablation: W = P * sV as bf16, [head][token]
  __shared__ __attribute__((aligned(16))) uint16_t s_wb[BPV ? 16 : 1][BPV ? kWbStride : 8];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int lg = lane >> 4, lr = lane & 15;
  const int p = blockIdx.x, kv = blockIdx.y, s = blockIdx.z;
  const int grp = a.group;
  const int Hkv = a.num_kv_heads;
  // MFMA rows: query qi of the sequence's nq (the newest nq positions), head
  // hg of the GQA group: row = qi * grp + hg (nq = 1: the group's heads)
  // (MQ = false: one query per sequence, the rows are the group's heads)
  const int nq = MQ ? a.nq : 1;
  const int rows = MQ ? grp * nq : grp;
  auto qrow = [&](int row) {  // [S * nq, Hq] index of a row's query
    const int qi = MQ ? row / grp : 0;
    return ((size_t)s * nq + qi) * a.num_q_heads + (size_t)kv * grp + (row - qi * grp);
  };

  // ---- first round trip: the sequence length, the block-table entries of the
  // pages this thread reads, the queries and their scales.  None of them
  // depends on another, so they are all in flight together.
  const int L_raw = a.seq_lens[s];
  if constexpr (MODE != kOneRound) {
    // In a grid of several rounds many workgroups lie past their sequence
    // (the grid is sized by max_seq_len): they leave on the length alone,
    // before issuing the loads below -- batch 16 at L ~ U[1K, 32K], 45% of
    // the 8000 workgroups: partition kernel 119.1 -> 113.7 us; one long
    // sequence (32K, all workgroups live) unchanged.  Partition 0 of an empty
    // sequence stays (it writes the zeros, or the fused step's outputs).
    const int Lc = min(max(L_raw, 0), a.max_seq_len);
    if (p >= max((Lc + kPartition - 1) / kPartition, 1)) return;
  }
  const int32_t* bt_row = a.block_tables + (size_t)s * a.max_blocks_per_seq;
  auto bt_at = [&](int j) { return bt_row[min(p * 16 + j, a.max_blocks_per_seq - 1)]; };
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const int tsv = tid & (kPartition - 1);  // V scale of token tsv (threads >= 256 repeat)
  int pidk[PPW], pidv[4];
#pragma unroll
  for (int j = 0; j < PPW; ++j) pidk[j] = bt_at(wu * PPW + j);  // K pages of this wave
#pragma unroll
  for (int g = 0; g < 4; ++g) pidv[g] = bt_at(4 * g + lg);      // V pages of this lane
  int pids = bt_at(tsv >> 4);
  v4i qa[NC];
  v4u qh[QB ? NC : 1][2];  // QB: bf16 dims 64c + 16lg + 8e .. +7 of row lr
  float sq[4];
  // Fused step: wave w quantizes items w, w + NW, ... of the group's grp q
  // heads followed by the newest token's K (item grp) and V (item grp + 1);
  // their bf16 inputs are part of this round trip.
  constexpr int kMaxItems = (16 + 2 + NW - 1) / NW;
  uint2 raw[kMaxItems];
  if constexpr (FUSED) {
#pragma unroll
    for (int k = 0; k < kMaxItems; ++k) {
      const int it = wu + k * NW;
      raw[k] = make_uint2(0u, 0u);
      if (it < grp)
        raw[k] = load_wave_vector<D>(
            a.new_query + ((size_t)s * a.num_q_heads + (size_t)kv * grp + it) * D, lane);
      else if (it < grp + 2)
        raw[k] = load_wave_vector<D>(
            (it == grp ? a.new_key : a.new_value) + ((size_t)s * Hkv + kv) * D, lane);
    }
  } else if constexpr (QB) {
    const bool vh = lr < rows;
    const uint16_t* qp = a.q_bf16 + qrow(vh ? lr : 0) * D + 16 * lg;
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        qh[c][e] = *reinterpret_cast<const v4u*>(qp + 64 * c + 8 * e);
        if (!vh) qh[c][e] = v4u{0u, 0u, 0u, 0u};
      }
#pragma unroll
    for (int r = 0; r < 4; ++r) sq[r] = 1.0f;
  } else {
    const bool vh = lr < rows;
    const int8_t* qp = a.q_int8 + qrow(vh ? lr : 0) * D + 16 * lg;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      qa[c] = *reinterpret_cast<const v4i*>(qp + 64 * c);
      if (!vh) qa[c] = v4i{0, 0, 0, 0};
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = 4 * lg + r;
      sq[r] = a.q_scale[qrow(min(h, rows - 1))];
      if (h >= rows) sq[r] = 0.0f;
    }
  }

  // keep the loads above ahead of the early exits below (the compiler would
  // otherwise sink them past the wait for the sequence length)
  asm volatile("" ::: "memory");

  // ---- second round trip: the scales and K bytes of the partition (V follows
  // once this wave's QK has consumed K, so V reuses its registers and K is not
  // queued behind V).  Entries past the sequence are clamped to a valid page:
  // what they load is discarded (scores of tokens >= L are -inf and their W
  // and scales are 0), so no load is conditional.  The fused step issues these
  // loads before its quantization, which then runs while they are in flight.
  auto clamp_page = [&](int pg) { return min(max(pg, 0), a.num_blocks - 1); };
  float sk[PPW];
  float sv_ld;
  v4i kb[PPW][NC];
  int pidv_raw[4];  // fused step: the table entries as read (the newest token's page is one)
  auto issue_k = [&]() {
    // K and V pages are read once per call: non-temporal loads (streaming
    // hint, no cache retention) -- 16K decode 13.8 -> 12.9 us, 32K 21.0 ->
    // 19.8 us, batch 16 136 -> 131 us against ordinary loads
#pragma unroll
    for (int j = 0; j < PPW; ++j) {
      const int8_t* base = a.k_cache + ((size_t)pidk[j] * Hkv + kv) * (size_t)(D / 16) * 256;
#pragma unroll
      for (int c = 0; c < NC; ++c)
        kb[j][c] = __builtin_nontemporal_load(
            reinterpret_cast<const v4i*>(base + (4 * c + lg) * 256 + lr * 16));
    }
  };
  auto issue_scales = [&]() {
    if constexpr (FUSED) {
#pragma unroll
      for (int g = 0; g < 4; ++g) pidv_raw[g] = pidv[g];
    }
#pragma unroll
    for (int g = 0; g < 4; ++g) pidv[g] = clamp_page(pidv[g]);
    pids = clamp_page(pids);
#pragma unroll
    for (int j = 0; j < PPW; ++j)
      sk[j] = a.k_scale[((size_t)pidk[j] * kBlockSize + lr) * Hkv + kv];
    sv_ld = a.v_scale[((size_t)pids * kBlockSize + (tsv & 15)) * Hkv + kv];
  };
  auto second_round_trip = [&]() {
#pragma unroll
    for (int j = 0; j < PPW; ++j) pidk[j] = clamp_page(pidk[j]);
    if constexpr (FUSED) {
      issue_scales();
      __builtin_amdgcn_sched_barrier(0);
      issue_k();
    } else {
      // The K addresses need only the wave-uniform (scalar) table entries:
      // K goes out before the wait for the per-lane V-page and scale-page
      // entries, the scales after it (16K partition kernel 9.63 -> 9.32 us,
      // 4K 7.71 -> 7.38 us, batch 16 call 119.7 -> 119.3 us, A/B in one
      // process).  The fused step keeps the scales first: with this order
      // its step measured 13.2 -> 13.6 us.
      issue_k();
      __builtin_amdgcn_sched_barrier(0);
      issue_scales();
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  const int L = min(max(L_raw, 0), a.max_seq_len);
  const int P_s = (L + kPartition - 1) / kPartition;
  if constexpr (FUSED) {
    // A partition past its sequence (a shorter sequence of a batch) has
    // nothing to do -- partition 0 still writes the query outputs and the
    // zeros of an empty sequence -- and leaves before issuing K loads it would
    // discard (batch 16 at L ~ U[1K, 32K]: fused step 141.4 -> 131.5 us).  The
    // length arrives with the block-table entries the K addresses need, so
    // this costs no extra wait; the exit comes before the loads rather than
    // around them so that every path past it has the same loads in flight
    // (with the loads in a branch the quantization below waited for all of
    // K: 16K step +0.8 us).
    if (p >= max(P_s, 1)) return;
    second_round_trip();
  }
  // a row's output element: fp32, or bf16 (nearest, ties to even)
  auto put_out = [&](int row, int dim, float v) {
    const size_t i = qrow(row) * D + dim;
    if (a.out16) a.out16[i] = (uint16_t)bf16_rne_bits(v);
    else a.out[i] = v;
  };
  // the newest token (position L - 1) lives in the sequence's last partition
  const bool newest_here = FUSED && L > 0 && p == P_s - 1;
  if constexpr (FUSED) {
    if (p < max(P_s, 1)) {
      constexpr int EPL = D / kWave;
#pragma unroll
      for (int k = 0; k < kMaxItems; ++k) {
        const int it = wu + k * NW;
        if (it >= grp + 2 || (it >= grp && !newest_here)) continue;  // wave-uniform
        float sc;
        const uint32_t codes = quantize_wave_vector<D>(raw[k], sc);
        int8_t* lds = it < grp ? s_q[it] : (it == grp ? s_nk : s_nv);
        if constexpr (EPL == 4) *reinterpret_cast<uint32_t*>(lds + lane * 4) = codes;
        else if constexpr (EPL == 2) *reinterpret_cast<uint16_t*>(lds + lane * 2) = (uint16_t)codes;
        else lds[lane] = (int8_t)codes;
        if (it < grp) {
          if (lane == 0) s_qs[it] = sc;
          if (p == 0 && a.q_int8_w) {  // the producer's Q outputs, written once
            const size_t qrow = (size_t)s * a.num_q_heads + (size_t)kv * grp + it;
            int8_t* dst = a.q_int8_w + qrow * D + lane * EPL;
            if constexpr (EPL == 4) *reinterpret_cast<uint32_t*>(dst) = codes;
            else if constexpr (EPL == 2) *reinterpret_cast<uint16_t*>(dst) = (uint16_t)codes;
            else *dst = (int8_t)codes;
            if (lane == 0) a.q_scale_w[qrow] = sc;
          }
        } else {
          // the producer's cache write of the newest token (slot from the table)
          if (lane == 0) s_nsc[it - grp] = sc;
          const int pos = L - 1;
          // page j of this partition's 16 was read in the first round trip by
          // the lanes of group j % 4, as entry j / 4 (no second table read,
          // whose wait would have included every load in flight)
          const int j = pos / kBlockSize - 16 * p;
          const int pv = j < 4 ? pidv_raw[0] : j < 8 ? pidv_raw[1] : j < 12 ? pidv_raw[2] : pidv_raw[3];
          const int blk = __builtin_amdgcn_readlane(pv, 16 * (j & 3));
          if (blk >= 0 && blk < a.num_blocks) {
            const int off = pos % kBlockSize;
            if (it == grp) store_k_token<D>(a.k_cache_w, blk, kv, Hkv, off, lane, codes);
            else store_v_token<D>(a.v_cache_w, blk, kv, Hkv, off, lane, codes);
            if (lane == 0)
              (it == grp ? a.k_scale_w : a.v_scale_w)[((size_t)blk * kBlockSize + off) * Hkv + kv] = sc;
          }
        }
      }
    }
  }
  if (L == 0) {
    if (p == 0 && a.stage == 0)
      for (int i = tid; i < rows * D; i += NT) put_out(i / D, i % D, 0.0f);
    return;
  }
  if (p >= P_s) return;
  // one partition and both stages in this call: the partition's output is the
  // sequence's output (w_0 o_0 / w_0); otherwise the partials go to the
  // workspace for the merge
  const bool direct = P_s == 1 && a.stage == 0;
  const int tok0 = p * kPartition;
  // per output row r of this lane (rows 4 lg + r): the causal key limit and
  // the output offset, computed once
  int vis[4];
  size_t obase[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int h = min(4 * lg + r, rows - 1);
    vis[r] = MQ ? L - nq + h / grp + 1 : L;
    obase[r] = qrow(h) * D;
  }
  if constexpr (!FUSED) second_round_trip();
#pragma unroll
  for (int j = 0; j < PPW; ++j)
    if (tok0 + 16 * (w * PPW + j) + lr >= L) sk[j] = 0.0f;
  if (tid < kPartition) s_sv[tid] = (tok0 + tid < L) ? sv_ld : 0.0f;

  const int t_new = L - 1 - tok0;  // newest token within the partition (if newest_here)
  if constexpr (FUSED) {
    __syncthreads();  // s_q, s_qs, s_nk, s_nv, s_nsc
#pragma unroll
    for (int c = 0; c < NC; ++c)
      qa[c] = lr < grp ? *reinterpret_cast<const v4i*>(&s_q[lr][64 * c + 16 * lg]) : v4i{0, 0, 0, 0};
#pragma unroll
    for (int r = 0; r < 4; ++r) sq[r] = 4 * lg + r < grp ? s_qs[4 * lg + r] : 0.0f;
    if (newest_here) {
      // this thread's K registers and V scale slot may hold the cache contents
      // from before the write above: use the new token's codes and scales
#pragma unroll
      for (int j = 0; j < PPW; ++j)
        if (16 * (w * PPW + j) + lr == t_new) {
#pragma unroll
          for (int c = 0; c < NC; ++c) kb[j][c] = *reinterpret_cast<const v4i*>(&s_nk[64 * c + 16 * lg]);
          sk[j] = s_nsc[0];
        }
      if (tid == t_new) s_sv[tid] = s_nsc[1];
    }
  }

  // ---- QK, the V loads, then scores -> LDS -------------------------------------
  v4i qk[PPW];
  v4f qkf[QB ? PPW : 1];
#pragma unroll
  for (int j = 0; j < PPW; ++j) {
    if constexpr (QB) {
      // the lane's 16 K bytes of chunk 4c + lg are dims 64c + 16lg .. +15: two
      // bf16 k-slices of 8, matched by the query halves qh[c][0], qh[c][1]
      qkf[j] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const v4u kw = __builtin_bit_cast(v4u, kb[j][c]);
        qkf[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(v8bf, qh[c][0]), i8x8_to_bf16(kw[0], kw[1]), qkf[j], 0, 0, 0);
        qkf[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(v8bf, qh[c][1]), i8x8_to_bf16(kw[2], kw[3]), qkf[j], 0, 0, 0);
      }
    } else {
      qk[j] = v4i{0, 0, 0, 0};
#pragma unroll
      for (int c = 0; c < NC; ++c)
        qk[j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(qa[c], kb[j][c], qk[j], 0, 0, 0);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  v4i vb[4][NCW];
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int8_t* base = a.v_cache + ((size_t)pidv[g] * Hkv + kv) * (size_t)D * 16;
#pragma unroll
    for (int c = 0; c < NCW; ++c)
      vb[g][c] = __builtin_nontemporal_load(
          reinterpret_cast<const v4i*>(base + (DecodeShape<D>::DW * w + 16 * c + lr) * 16));
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < PPW; ++j) {
    const int tl = 16 * (w * PPW + j) + lr;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = 4 * lg + r;
      if (h < rows) {
        float x = QB ? qkf[j][r] : (float)qk[j][r] * sq[r];
        x = x * sk[j];
        x = x * a.softmax_scale;
        // causal: query qi sits at position L - nq + qi and sees keys up to it
        s_sc[h * kTokStride + tl] = (tok0 + tl < vis[r]) ? x : -INFINITY;
      }
    }
  }
  __syncthreads();

  // ---- softmax and W quantization: wave h owns head h, lane l tokens 4l..4l+3
  for (int h = w; h < rows; h += NW) {
    const float4 x4 = *reinterpret_cast<const float4*>(&s_sc[h * kTokStride + 4 * lane]);
    const float x[4] = {x4.x, x4.y, x4.z, x4.w};
    float m = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    m = group_max<kWave>(m);
    float e[4];
    double ls = 0.0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      e[i] = (x[i] == -INFINITY) ? 0.0f : exp_f32_rn(x[i] - m);
      ls += (double)e[i];
    }
    ls = group_sum<kWave>(ls);
    const float l = (float)ls;
    // l >= 1 (the max term is exp(0) = 1), or 0 for a row that sees no token
    // of this partition (later queries' keys): then P = W = 0, m = -inf
    const double rl = l > 0.0f ? rcp_f64((double)l) : 0.0;
    const float4 v4 = *reinterpret_cast<const float4*>(&s_sv[4 * lane]);
    const float sv[4] = {v4.x, v4.y, v4.z, v4.w};
    float W[4];
    float am = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float P = l > 0.0f ? div_f32_rn(e[i], l, rl) : 0.0f;  // == e / l (IEEE)
      W[i] = P * sv[i];
      am = fmaxf(am, W[i]);
    }
    if constexpr (BPV) {
      // the ablation: W itself, rounded to bf16, no group quantization
      const uint32_t lo = bf16_rne_bits(W[0]) | (bf16_rne_bits(W[1]) << 16);
      const uint32_t hi = bf16_rne_bits(W[2]) | (bf16_rne_bits(W[3]) << 16);
      *reinterpret_cast<uint2*>(&s_wb[h][4 * lane]) = make_uint2(lo, hi);
      if (lane == 0) {
        s_M[h] = m;
        s_L[h] = l;
      }
      continue;
    }
    am = group_max<G / 4>(am);  // G consecutive tokens = G/4 consecutive lanes
    // == am / 127 (IEEE), or am / 255 for UINT8 W
    const float sw = U8W ? div_f32_rn(am, 255.0f, 1.0 / 255.0) : div_f32_rn(am, 127.0f, 1.0 / 127.0);
    // UINT8 codes c in [0, 255] are stored as c - 128 (int8); the PV adds
    // 128 * (sum of the group's V) back
    uint32_t packed = U8W ? 0x80808080u : 0u;
    if (sw > 0.0f) {  // sW = 0 (also when max W / 127 underflows): the group adds 0
      const double rsw = rcp_f64((double)sw);
      packed = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float q = div_f32_rn(W[i], sw, rsw);
        const uint32_t c = U8W ? (uint32_t)(fminf(roundf(q), 255.0f)) ^ 0x80u : (uint32_t)round_code(q);
        packed |= (c & 0xff) << (8 * i);
      }
    }
    *reinterpret_cast<uint32_t*>(&s_wq[h * kWqStride + 4 * lane]) = packed;
    if (((4 * lane) & (G - 1)) == 0) s_sw[h][(4 * lane) / G] = sw;
    if (lane == 0) {
      s_M[h] = m;
      s_L[h] = l;
    }
  }
  __syncthreads();

  if (FUSED && newest_here) {
    // V bytes of the newest token (byte t_new % 16 of the 16-token rows of
    // page t_new / 16) from the codes quantized above
#pragma unroll
    for (int g = 0; g < 4; ++g)
      if (4 * g + lg == t_new / 16) {
        const int bsel = t_new % 16;
#pragma unroll
        for (int c = 0; c < NCW; ++c) {
          const uint32_t code = (uint8_t)s_nv[DecodeShape<D>::DW * w + 16 * c + lr];
          const uint32_t word = (uint32_t)vb[g][c][bsel >> 2];
          const int sh = 8 * (bsel & 3);
          vb[g][c][bsel >> 2] = (int)((word & ~(0xffu << sh)) | (code << sh));
        }
      }
  }

  // ---- PV ------------------------------------------------------------------------
  float o[NCW][4];
#pragma unroll
  for (int c = 0; c < NCW; ++c)
#pragma unroll
    for (int r = 0; r < 4; ++r) o[c][r] = 0.0f;
  const v4i zero = {0, 0, 0, 0};
  if constexpr (BPV) {
    // v_mfma_f32_16x16x32_bf16: lane group lg supplies the same 8 tokens to
    // both operands -- half hf of page 4g + lg -- so each MFMA sums 32 tokens
    v4f acc[NCW];
#pragma unroll
    for (int c = 0; c < NCW; ++c) acc[c] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int g = 0; g < 4; ++g) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        v4u wa = v4u{0u, 0u, 0u, 0u};
        if (lr < rows) wa = *reinterpret_cast<const v4u*>(&s_wb[lr][16 * (4 * g + lg) + 8 * hf]);
        const v8bf A = __builtin_bit_cast(v8bf, wa);
#pragma unroll
        for (int c = 0; c < NCW; ++c) {
          const v8bf B = i8x8_to_bf16((uint32_t)vb[g][c][2 * hf], (uint32_t)vb[g][c][2 * hf + 1]);
          acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B, acc[c], 0, 0, 0);
        }
      }
    }
#pragma unroll
    for (int c = 0; c < NCW; ++c)
#pragma unroll
      for (int r = 0; r < 4; ++r) o[c][r] = acc[c][r];
  }
#pragma unroll
  for (int g = 0; g < (BPV ? 0 : 4); ++g) {
    const v4i wa = lr < rows ? *reinterpret_cast<const v4i*>(&s_wq[lr * kWqStride + 64 * g + 16 * lg])
                            : zero;
    float s0[4], s1[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = min(4 * lg + r, 15);
      s0[r] = G == 64 ? s_sw[h][g] : s_sw[h][(2 * g) % NGP];
      s1[r] = G == 64 ? 0.0f : s_sw[h][(2 * g + 1) % NGP];
    }
    // UINT8 W: all-ones A rows give each group's V column sums (masked like W)
    const v4i ones = {0x01010101, 0x01010101, 0x01010101, 0x01010101};
#pragma unroll
    for (int c = 0; c < NCW; ++c) {
      if constexpr (G == 64) {
        v4i acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(wa, vb[g][c], zero, 0, 0, 0);
        if constexpr (U8W) {
          const v4i cs = __builtin_amdgcn_mfma_i32_16x16x64_i8(ones, vb[g][c], zero, 0, 0, 0);
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[r] += cs[r] << 7;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) o[c][r] += s0[r] * (float)acc[r];
      } else {
        v4i alo = __builtin_amdgcn_mfma_i32_16x16x64_i8(lg < 2 ? wa : zero, vb[g][c], zero,
                                                        0, 0, 0);
        v4i ahi = __builtin_amdgcn_mfma_i32_16x16x64_i8(lg < 2 ? zero : wa, vb[g][c], zero,
                                                        0, 0, 0);
        if constexpr (U8W) {
          const v4i clo = __builtin_amdgcn_mfma_i32_16x16x64_i8(lg < 2 ? ones : zero, vb[g][c],
                                                                zero, 0, 0, 0);
          const v4i chi = __builtin_amdgcn_mfma_i32_16x16x64_i8(lg < 2 ? zero : ones, vb[g][c],
                                                                zero, 0, 0, 0);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            alo[r] += clo[r] << 7;
            ahi[r] += chi[r] << 7;
          }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          o[c][r] += s0[r] * (float)alo[r];
          o[c][r] += s1[r] * (float)ahi[r];
        }
      }
    }
  }

  // ---- output (single partition) or partial --------------------------------------
  const size_t node = (((size_t)s * Hkv + kv) * a.max_parts + p) * rows;
  if (!direct && MODE == kRoundsNt) {
    // The workgroup's partials are one contiguous rows x D block: staged in
    // the score tile (free since the softmax) and written as 16-byte
    // non-temporal stores (batch 16 at L ~ U[1K, 32K]: partition kernel 113.8
    // -> 110.8 us, 32K 15.4 -> 15.2 us; with 512-byte partials, the MHA
    // batch, the barrier costs more than it saves: 98.0 against 99.0 us).
    float* stage = s_sc;
#pragma unroll
    for (int c = 0; c < NCW; ++c) {
      const int dim = DecodeShape<D>::DW * w + 16 * c + lr;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int h = 4 * lg + r;
        if (h < rows) stage[h * D + dim] = o[c][r];
      }
    }
    __syncthreads();
    v4f* dst = reinterpret_cast<v4f*>(a.part_o + node * D);
    for (int i = tid; i < rows * D / 4; i += NT)
      __builtin_nontemporal_store(reinterpret_cast<const v4f*>(stage)[i], dst + i);
  } else {
#pragma unroll
    for (int c = 0; c < NCW; ++c) {
      const int dim = DecodeShape<D>::DW * w + 16 * c + lr;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int h = 4 * lg + r;
        if (h < rows) {
          if (direct) {
            if (a.out16) a.out16[obase[r] + dim] = (uint16_t)bf16_rne_bits(o[c][r]);
            else a.out[obase[r] + dim] = o[c][r];
          } else {
            a.part_o[(node + h) * D + dim] = o[c][r];
          }
        }
      }
    }
  }
  if (!direct && tid < rows) {
    float* ml = a.part_ml + (node + tid) * 2;
    if constexpr (MODE == kRoundsNt) {
      __builtin_nontemporal_store(s_M[tid], ml);
      __builtin_nontemporal_store(s_L[tid], ml + 1);
    } else {
      ml[0] = s_M[tid];
      ml[1] = s_L[tid];
    }
  }
}

// One wave per (q head, sequence, 32-dim slice), no barriers:
//   O = sum_p w_p o_p / sum_p w_p, w_p = l_p exp(m_p - M), M = max_p m_p.
// Lane l owns float4 column l % 8 of the 32-dim slice for partitions
// p = l / 8 (mod 8), U per round (RP = 8 U partitions per round: 64, or 128
// when the call has more than 64); for a single sequence the partial loads of
// the first round and the (m, l) of partitions l, l + 64, ... of the first
// round go out before the sequence length is known (every slot below
// max_parts exists in the workspace; slots past the sequence are discarded),
// so a sequence of up to RP partitions costs one memory round trip.  The weight of partition p is
// computed by lane p % 64 and fetched with a cross-lane read; the eight lane
// groups are summed with two swaps and one xor exchange.  (32 rather than 64
// dims per wave: twice the waves, half the loads per lane -- 1% faster at
// 16K, 1.2% at 32K.)  Every lane adds its partitions in increasing order
// whatever U is, so U does not change the result.
template <int D, int U>
__global__ __launch_bounds__(kWave) void paged_decode_merge_kernel(DecodeArgs a) {
  constexpr int RP = 8 * U;        // partitions per round
  constexpr int NML = RP / kWave;  // (m, l) pairs per lane per round
  static_assert(RP % kWave == 0, "a round covers whole waves of partitions");
  // blockIdx.x = qi * Hq + h: query qi (of nq) of the sequence, q head h
  const int qi = blockIdx.x / a.num_q_heads, h = blockIdx.x % a.num_q_heads;
  const int s = blockIdx.y, slice = blockIdx.z, lane = threadIdx.x;
  const int grp = a.group, rows = grp * a.nq;
  const int kv = h / grp, row = qi * grp + h % grp;
  const size_t base = ((size_t)s * a.num_kv_heads + kv) * a.max_parts;
  const float2* ml = reinterpret_cast<const float2*>(a.part_ml) + base * rows + row;
  const int col = lane & 7, lg = lane >> 3;
  const size_t ostride = (size_t)rows * D;
  const float* po = a.part_o + (base * rows + row) * D + 32 * slice + 4 * col;
  float4 v[U];
  int qlast = a.max_parts - 1;
  auto issue = [&](int q0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int q = min(q0 + lg + 8 * u, qlast);
      v[u] = *reinterpret_cast<const float4*>(po + (size_t)q * ostride);
    }
  };
  float2 ml0[NML];
  auto issue_first = [&]() {
    issue(0);
#pragma unroll
    for (int k = 0; k < NML; ++k) ml0[k] = ml[(size_t)min(lane + kWave * k, qlast) * rows];
  };
  // One sequence: the first round goes out before its length is known (one
  // memory round trip).  A batch waits for the length and loads no slot past
  // its sequence, so that its shorter sequences do not fetch what they drop
  // (with U = 16: batch 16 at L ~ U[1K, 32K] call 123.6 -> 123.0 us, MHA
  // batch 8 102.4 -> 101.9 us, A/B in one process).
  int L = a.seq_lens[s];
  const bool batch = a.num_seqs > 1;
  if (!batch) issue_first();
  L = min(max(L, 0), a.max_seq_len);
  const int P_s = (L + kPartition - 1) / kPartition;
  if (batch) {
    qlast = max(P_s - 1, 0);
    if (!(a.stage == 0 && P_s <= 1)) issue_first();
  }
  const size_t o = (((size_t)s * a.nq + qi) * a.num_q_heads + h) * D + 32 * slice;
  auto put4 = [&](float x0, float x1, float x2, float x3) {
    if (a.out16)
      reinterpret_cast<uint2*>(a.out16 + o)[lane] =
          make_uint2(bf16_rne_bits(x0) | (bf16_rne_bits(x1) << 16),
                     bf16_rne_bits(x2) | (bf16_rne_bits(x3) << 16));
    else
      reinterpret_cast<float4*>(a.out + o)[lane] = make_float4(x0, x1, x2, x3);
  };
  if (a.stage == 0 && P_s <= 1) return;  // written by the partition kernel
  if (P_s <= 1) {
    // the merge alone: an empty sequence gives zeros, one partition its own
    // output (what the partition kernel writes when it runs both stages)
    if (lane < 8) {
      if (P_s == 0) put4(0.f, 0.f, 0.f, 0.f);
      else put4(v[0].x, v[0].y, v[0].z, v[0].w);
    }
    return;
  }

  float m = -INFINITY;
#pragma unroll
  for (int k = 0; k < NML; ++k)
    if (lane + kWave * k < P_s) m = fmaxf(m, ml0[k].x);
  for (int q = lane + RP; q < P_s; q += kWave) m = fmaxf(m, ml[(size_t)q * rows].x);
  const float M = group_max<kWave>(m);

  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float wsum = 0.0f;
  for (int q0 = 0; q0 < P_s; q0 += RP) {
    float wl[NML];  // weight of partition q0 + lane + 64 k
#pragma unroll
    for (int k = 0; k < NML; ++k) {
      const int q = q0 + lane + kWave * k;
      wl[k] = 0.0f;
      if (q < P_s) {
        const float2 e = q0 == 0 ? ml0[k] : ml[(size_t)q * rows];
        wl[k] = e.y > 0.0f ? e.y * expf(e.x - M) : 0.0f;  // l = 0: a partition this query does not see
      }
      wsum += wl[k];
    }
    // every weight this lane needs, fetched before any is used (one wait
    // for all the cross-lane reads instead of one per partition group)
    float wqs[U];
#pragma unroll
    for (int u = 0; u < U; ++u) wqs[u] = __shfl(wl[(8 * u) / kWave], (lg + 8 * u) % kWave, kWave);
    __builtin_amdgcn_sched_barrier(0);
    if (q0 > 0) issue(q0);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      // Slots of partitions past the sequence were loaded (before L was
      // known) but never written: whatever they hold, even NaN or Inf, is
      // dropped by the select, not multiplied by a zero weight.
      const bool live = q0 + lg + 8 * u < P_s;
      const float wq = wqs[u];
      acc.x += live ? wq * v[u].x : 0.0f;
      acc.y += live ? wq * v[u].y : 0.0f;
      acc.z += live ? wq * v[u].z : 0.0f;
      acc.w += live ? wq * v[u].w : 0.0f;
    }
  }
  wsum = group_sumf<kWave>(wsum);
  float r[4] = {acc.x, acc.y, acc.z, acc.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t x0, x1;
    swap16(f_bits(r[i]), x0, x1);
    r[i] = bits_f(x0) + bits_f(x1);
    swap32(f_bits(r[i]), x0, x1);
    r[i] = bits_f(x0) + bits_f(x1);
    r[i] += __shfl_xor(r[i], 8, kWave);
  }
  if (lane < 8) {
    // wsum = 0 only for a query that sees no key at all (seq_len < nq): zeros
    const float inv = wsum > 0.0f ? 1.0f / wsum : 0.0f;
    put4(r[0] * inv, r[1] * inv, r[2] * inv, r[3] * inv);
  }
}

// The merge with one round per 64 partitions (U = 8) or per 128 (U = 16),
// the wider round whenever a sequence may have more than 64 partitions (32K:
// 20.4 -> 19.9 us per call; in a batch it pays once the first round no longer
// loads slots past each sequence).
template <int D>
void launch_merge(const DecodeArgs& a, dim3 mgrid, hipStream_t stream) {
  if (a.max_parts > 64)
    hipLaunchKernelGGL((paged_decode_merge_kernel<D, 16>), mgrid, dim3(kWave), 0, stream, a);
  else
    hipLaunchKernelGGL((paged_decode_merge_kernel<D, 8>), mgrid, dim3(kWave), 0, stream, a);
}

// Grids of more workgroups than the chip has CUs (256) run in several
// rounds (kRounds).  When each workgroup also writes kilobytes of partials,
// the plain and fused int8 kernels store them with the non-temporal hint
// (kRoundsNt; A/B in one process: batch 16 at L ~ U[1K, 32K], 6 KB per
// workgroup, partition kernel 123.3 -> 119.2 us; 32K call 19.22 -> 18.99 us).
// A grid of one round keeps ordinary stores (16K: 9.63 against 9.84 us with
// the hint), and so do small partials (the MHA batch, 512 B per workgroup:
// 100.5 against 101.3 us).
constexpr int64_t kRoundsMinGroups = 257;
constexpr int64_t kNtPartialsMinBytes = 4096;

hipError_t launch_paged_decode(const DecodeArgs& a, hipStream_t stream) {
  if (a.num_seqs == 0) return hipSuccess;
  const bool rounds = (int64_t)a.max_parts * a.num_kv_heads * a.num_seqs >= kRoundsMinGroups;
  const bool ntp =
      rounds && (int64_t)a.group * a.nq * a.head_dim * (int64_t)sizeof(float) >= kNtPartialsMinBytes;
  dim3 grid((unsigned)a.max_parts, (unsigned)a.num_kv_heads, (unsigned)a.num_seqs);
  dim3 mgrid((unsigned)(a.num_q_heads * a.nq), (unsigned)a.num_seqs, (unsigned)(a.head_dim / 32));
#define I8KV_DECODE_CASE(DD, GG)                                                                 \
  if (a.head_dim == DD && (a.pv_bf16 ? GG == 64 : a.w_group == GG)) {                            \
    const dim3 blk(DecodeShape<DD>::NW * kWave);                                                 \
    const bool mq = a.nq > 1;                                                                    \
    if (a.stage == 2) {                                                                          \
      launch_merge<DD>(a, mgrid, stream);                                                        \
      return hipGetLastError();                                                                  \
    }                                                                                            \
    if (a.new_key && ntp)                                                                        \
      hipLaunchKernelGGL((paged_decode_partition_kernel<DD, GG, true, kPvInt8, false, false, kRoundsNt>), \
                         grid, blk, 0, stream, a);                                               \
    else if (a.new_key && rounds)                                                                \
      hipLaunchKernelGGL((paged_decode_partition_kernel<DD, GG, true, kPvInt8, false, false, kRounds>), \
                         grid, blk, 0, stream, a);                                               \
    else if (a.new_key)                                                                          \
      hipLaunchKernelGGL((paged_decode_partition_kernel<DD, GG, true, kPvInt8, false, false>),   \
                         grid, blk, 0, stream, a);                                               \
    else if (a.q_bf16)                                                                           \
      hipLaunchKernelGGL((paged_decode_partition_kernel<DD, GG, false, kPvInt8, false, true>),   \
                         grid, blk, 0, stream, a);                                               \
    else if (a.pv_bf16 && mq)                                                                    \
      hipLaunchKernelGGL((paged_decode_partition_kernel<DD, GG, false, kPvBf16, true, false>),   \
                         grid, blk, 0, stream, a);                                               \
    else if (a.pv_bf16)                                                                          \
      hipLaunchKernelGGL((paged_decode_partition_kernel<DD, GG, false, kPvBf16, false, false>),  \
                         grid, blk, 0, stream, a);                                               \
    else if (a.w_uint8 && mq)                                                                    \
      hipLaunchKernelGGL((paged_decode_partition_kernel<DD, GG, false, kPvUint8, true, false>),  \
                         grid, blk, 0, stream, a);                                               \
    else if (a.w_uint8)                                                                          \
      hipLaunchKernelGGL((paged_decode_partition_kernel<DD, GG, false, kPvUint8, false, false>), \
                         grid, blk, 0, stream, a);                                               \
    else if (mq && rounds)                                                                       \
      hipLaunchKernelGGL((paged_decode_partition_kernel<DD, GG, false, kPvInt8, true, false, kRounds>), \
                         grid, blk, 0, stream, a);                                               \
    else if (mq)                                                                                 \
      hipLaunchKernelGGL((paged_decode_partition_kernel<DD, GG, false, kPvInt8, true, false>),   \
                         grid, blk, 0, stream, a);                                               \
    else if (ntp)                                                                                \
      hipLaunchKernelGGL((paged_decode_partition_kernel<DD, GG, false, kPvInt8, false, false, kRoundsNt>), \
                         grid, blk, 0, stream, a);                                               \
    else if (rounds)                                                                             \
      hipLaunchKernelGGL((paged_decode_partition_kernel<DD, GG, false, kPvInt8, false, false, kRounds>), \
                         grid, blk, 0, stream, a);                                               \
    else                                                                                         \
      hipLaunchKernelGGL((paged_decode_partition_kernel<DD, GG, false, kPvInt8, false, false>),  \
                         grid, blk, 0, stream, a);                                               \
    if (a.max_parts > 1 && a.stage == 0)                                                         \
      launch_merge<DD>(a, mgrid, stream);                                                        \
    return hipGetLastError();                                                                    \
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
