// MLA attention over the FP8 latent cache: paged decode (with MTP query tokens) and
// sparse MLA over indexer-selected tokens.
//
// Sources: vLLM AgentX article (news.ainew.jp), "Kimi K3" (MLA keeps one latent head;
// partial outputs merged by log-sum-exp) and "DeepSeek V4" (sparse MLA gathers the top-k
// KV entries, then attends); GLM-5.3 report (aisoku.org), "What's new" (the latent KV is
// shared by all 64 heads), its table (FP8 KV, MTP3) and "How to try" (prompts inside the
// top-k use the same sparse MQA kernel).
//
// The latent is shared by every query head, so attention is MQA with d_qk = 576 (512
// latent + 64 rope) and d_v = 512 (the latent itself).  A workgroup owns 64 query rows
// (4 waves x 16 rows) that read the same keys: 64 heads of one query token.  Each
// 32-key tile is staged once in LDS for all 64 rows:
//   * keys are gathered through the block table (decode: a contiguous key range;
//     sparse: the query's selected positions), 4 tokens x 16 bytes per thread;
//   * FP8 E4M3 is upcast exactly (hardware converter) to bf16, stored row-major for the
//     QK operand (queries are bf16), and to fp16, stored transposed (dims x keys) for
//     the PV operand (P in fp16 keeps 11 significant bits);
//   * the per-token fp32 scale is folded into the scores (s = scale_t * q.k) and into
//     the probabilities used for PV (p * scale_t), never into the stored bf16;
//   * S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (Q^T in registers, 18 k-steps), online
//     softmax on the C tile (one query row per lane), O^T += V^T P^T
//     (v_mfma_f32_16x16x32_f16) with the probabilities fed from registers.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kDqk = 576, kDv = 512, kBs = 64;
constexpr int kKT = 32;                   // keys per tile
constexpr int kKStride = kDqk + 8;        // bf16 per K row in LDS (1168 B)
constexpr int kVtStride = kKT + 8;        // bf16 per V^T row (80 B)
constexpr int kQS = kDqk / 32;            // 18 QK k-steps
constexpr int kMT = kDv / 16;             // 32 O^T tiles

struct MlaSmem {
  uint16_t k[kKT * kKStride];
  uint16_t vt[kDv * kVtStride];
  float ks[kKT];      // scale_t * softmax scale * log2(e), 0 for invalid keys
  float vs[kKT];      // scale_t
  int32_t kidx[kKT];  // logical position of the key, -1 if invalid
};

template <bool SPARSE>
__global__ __launch_bounds__(256, 1) void mla_kernel(MlaDecodeArgs da, SparseMlaArgs sa) {
  __shared__ __attribute__((aligned(16))) MlaSmem sm;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int m16 = lane & 15, grp = lane >> 4;

  // ---- work unit
  const uint16_t* qbase;
  const uint8_t* kv;
  const float* kv_scale;
  const int32_t* bt_row;
  const int32_t* sel = nullptr;   // sparse: selected positions
  int Hq, num_blocks, n_keys, k_begin = 0, n_lblocks, L = 0, T = 1, row0;
  float scale_log2;
  int unit_seq = 0, unit_split = 0;
  if constexpr (SPARSE) {
    Hq = sa.num_q_heads;
    const int rblocks = (Hq + 63) / 64;
    const int logical = blockIdx.x;
    const int i = logical / rblocks;
    row0 = (logical % rblocks) * 64;
    const int seq = sa.q_seq[i];
    qbase = sa.q + (size_t)i * Hq * kDqk;
    kv = sa.kv; kv_scale = sa.kv_scale; num_blocks = sa.num_blocks;
    bt_row = sa.bt + (size_t)seq * sa.bt_stride;
    sel = sa.topk + (size_t)i * sa.k;
    n_keys = sa.k;
    n_lblocks = sa.bt_stride;
    scale_log2 = sa.scale_log2;
    unit_seq = i;
  } else {
    Hq = da.num_q_heads;
    T = da.q_per_seq;
    const int rows = T * Hq;
    const int rblocks = (rows + 63) / 64;
    const int n_units = da.num_seqs * da.max_splits * rblocks;
    const int logical = xcd_swizzle(blockIdx.x, n_units);
    const int rb = logical % rblocks;
    unit_split = (logical / rblocks) % da.max_splits;
    unit_seq = logical / (rblocks * da.max_splits);
    row0 = rb * 64;
    L = min(da.context_len[unit_seq], da.max_context_len);
    k_begin = unit_split * kDecodeSplitMla;
    if (k_begin >= L) return;
    n_keys = min(L - k_begin, kDecodeSplitMla);
    qbase = da.q + (size_t)unit_seq * rows * kDqk;
    kv = da.kv; kv_scale = da.kv_scale; num_blocks = da.num_blocks;
    bt_row = da.bt + (size_t)unit_seq * da.bt_stride;
    n_lblocks = (L + kBs - 1) / kBs;
    scale_log2 = da.scale_log2;
  }
  const int rows_total = SPARSE ? Hq : T * Hq;

  // ---- this lane's query row: wave w owns rows row0 + 16w .. +15; C column = lane%16
  const int row = row0 + wave * 16 + m16;
  const bool row_ok = row < rows_total;
  const int row_c = row_ok ? row : rows_total - 1;
  const int pos = SPARSE ? 0x7fffffff : (L - T + row_c / Hq);
  u32x4 qb[kQS];
  {
    const uint16_t* qp = qbase + (size_t)row_c * kDqk + 8 * grp;
#pragma unroll
    for (int ks = 0; ks < kQS; ++ks) qb[ks] = ld16(qp + 32 * ks);
  }
  f32x4 acc[kMT];
#pragma unroll
  for (int mt = 0; mt < kMT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  for (int kb = 0; kb < n_keys; kb += kKT) {
    __syncthreads();
    // ---- gather the tile: key metadata, then 4 keys x 16 dims per group
    if (tid < kKT) {
      const int j = kb + tid;
      int idx = -1, pb = -1;
      if (j < n_keys) {
        idx = SPARSE ? sel[j] : k_begin + j;
        if (idx >= 0) pb = phys_block(bt_row, idx / kBs, n_lblocks, num_blocks);
      }
      const bool ok = pb >= 0;
      const float sc = ok ? kv_scale[(size_t)pb * kBs + idx % kBs] : 0.f;
      sm.kidx[tid] = ok ? idx : -1;
      sm.ks[tid] = sc * scale_log2;
      sm.vs[tid] = sc;
    }
    for (int gi = tid; gi < (kKT / 4) * (kDqk / 16); gi += 256) {
      const int kg = gi % (kKT / 4), dc = gi / (kKT / 4);
      u32x4 raw[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = kb + 4 * kg + e;
        int idx = -1, pb = -1;
        if (j < n_keys) {
          idx = SPARSE ? sel[j] : k_begin + j;
          if (idx >= 0) pb = phys_block(bt_row, idx / kBs, n_lblocks, num_blocks);
        }
        raw[e] = pb >= 0 ? ld16(kv + ((size_t)pb * kBs + idx % kBs) * kDqk + 16 * dc) : u32x4{0, 0, 0, 0};
      }
      // upcast 4 dims at a time: c[e] holds dims 16dc + 4w4 .. +3 of key 4kg+e
#pragma unroll
      for (int w4 = 0; w4 < 4; ++w4) {
        u32x2 c[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          c[e] = fp8x4_to_bf16x4(raw[e][w4]);
          *reinterpret_cast<u32x2*>(sm.k + (4 * kg + e) * kKStride + 16 * dc + 4 * w4) = c[e];
        }
        if (dc < kDv / 16) {
          uint16_t* vrow = sm.vt + (16 * dc + 4 * w4) * kVtStride + 4 * kg;
#pragma unroll
          for (int e = 0; e < 4; ++e) c[e] = fp8x4_to_f16x4(raw[e][w4]);
          u32x2 t;
          t.x = __builtin_amdgcn_perm(c[1].x, c[0].x, 0x05040100u);
          t.y = __builtin_amdgcn_perm(c[3].x, c[2].x, 0x05040100u);
          *reinterpret_cast<u32x2*>(vrow) = t;
          t.x = __builtin_amdgcn_perm(c[1].x, c[0].x, 0x07060302u);
          t.y = __builtin_amdgcn_perm(c[3].x, c[2].x, 0x07060302u);
          *reinterpret_cast<u32x2*>(vrow + kVtStride) = t;
          t.x = __builtin_amdgcn_perm(c[1].y, c[0].y, 0x05040100u);
          t.y = __builtin_amdgcn_perm(c[3].y, c[2].y, 0x05040100u);
          *reinterpret_cast<u32x2*>(vrow + 2 * kVtStride) = t;
          t.x = __builtin_amdgcn_perm(c[1].y, c[0].y, 0x07060302u);
          t.y = __builtin_amdgcn_perm(c[3].y, c[2].y, 0x07060302u);
          *reinterpret_cast<u32x2*>(vrow + 3 * kVtStride) = t;
        }
      }
    }
    __syncthreads();
    // ---- S^T = K Q^T for two 16-key sub-tiles
    f32x4 sacc[2];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      sacc[st] = f32x4{0.f, 0.f, 0.f, 0.f};
      const uint16_t* kp = sm.k + (16 * st + m16) * kKStride + 8 * grp;
#pragma unroll
      for (int ks = 0; ks < kQS; ++ks)
        sacc[st] = mfma16x16x32(*reinterpret_cast<const u32x4*>(kp + 32 * ks), qb[ks], sacc[st]);
    }
    // ---- scale, mask, online softmax; lane holds row `row`, keys 16st + 4grp + i
    float mx = -INFINITY;
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = 16 * st + 4 * grp + i;
        const int idx = sm.kidx[key];
        const bool ok = idx >= 0 && idx <= pos;
        const float v = ok ? sacc[st][i] * sm.ks[key] : -INFINITY;
        sacc[st][i] = v;
        mx = fmaxf(mx, v);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    float alpha = 1.f, rs = 0.f;
    u32x4 pb;
    if (m_new != -INFINITY) {
      alpha = fast_exp2(m_run - m_new);
      float pv[8];
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = fast_exp2(sacc[st][i] - m_new);
          rs += p;
          pv[4 * st + i] = p * sm.vs[16 * st + 4 * grp + i];
        }
      pb = u32x4{pack_f16x2(pv[0], pv[1]), pack_f16x2(pv[2], pv[3]),
                 pack_f16x2(pv[4], pv[5]), pack_f16x2(pv[6], pv[7])};
    } else {
      pb = u32x4{0, 0, 0, 0};
    }
    l_run = l_run * alpha + rs;
    m_run = m_new;
    // ---- O^T = alpha O^T + V^T P^T (keys 4grp..+3 and 16+4grp..+3 in register order)
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt) {
      const uint16_t* vp = sm.vt + (16 * mt + m16) * kVtStride + 4 * grp;
      const u32x2 lo = *reinterpret_cast<const u32x2*>(vp);
      const u32x2 hi = *reinterpret_cast<const u32x2*>(vp + 16);
      acc[mt] = mfma16x16x32_f16(u32x4{lo.x, lo.y, hi.x, hi.y}, pb, acc[mt] * alpha);
    }
  }

  // ---- finish: full row sum over the 4 lane groups, write
  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
  if (!row_ok) return;
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const float lse2 = l_tot > 0.f ? m_run + __log2f(l_tot) : -INFINITY;
  if constexpr (SPARSE) {
    uint16_t* op = sa.out + ((size_t)unit_seq * Hq + row) * kDv;
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt) {
      u32x2 w;
      w.x = pack_bf16x2(acc[mt][0] * inv, acc[mt][1] * inv);
      w.y = pack_bf16x2(acc[mt][2] * inv, acc[mt][3] * inv);
      *reinterpret_cast<u32x2*>(op + 16 * mt + 4 * grp) = w;
    }
    if (sa.lse != nullptr && grp == 0) sa.lse[(size_t)unit_seq * Hq + row] = lse2 == -INFINITY ? -INFINITY : lse2 * kLn2;
  } else {
    const size_t pbase = ((size_t)unit_seq * da.max_splits + unit_split) * rows_total + row;
    float* op = da.part_o + pbase * kDv;
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt)
      *reinterpret_cast<f32x4*>(op + 16 * mt + 4 * grp) = acc[mt] * inv;
    if (grp == 0) da.part_lse[pbase] = lse2;
  }
}

}  // namespace

hipError_t launch_mla_decode(const MlaDecodeArgs& a, hipStream_t stream) {
  const int rows = a.q_per_seq * a.num_q_heads;
  const unsigned grid = (unsigned)a.num_seqs * a.max_splits * ((rows + 63) / 64);
  if (grid == 0) return hipSuccess;
  SparseMlaArgs none{};
  hipLaunchKernelGGL((mla_kernel<false>), dim3(grid), dim3(256), 0, stream, a, none);
  return hipGetLastError();
}

hipError_t launch_sparse_mla(const SparseMlaArgs& a, hipStream_t stream) {
  const unsigned grid = (unsigned)a.n_q * ((a.num_q_heads + 63) / 64);
  if (grid == 0) return hipSuccess;
  MlaDecodeArgs none{};
  hipLaunchKernelGGL((mla_kernel<true>), dim3(grid), dim3(256), 0, stream, none, a);
  return hipGetLastError();
}

}  // namespace pa
