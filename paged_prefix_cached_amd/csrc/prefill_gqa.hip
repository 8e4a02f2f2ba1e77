// Prefix-cached suffix prefill over a paged bf16 pool (GQA / MHA, block size 16).
//
// Sources: vLLM AgentX article (news.ainew.jp), "Re-evaluating agentic workloads" (each
// turn re-sends the history; most of it is a cached prefix, the new prefill is short)
// and "Hybrid KV cache management" (one shared block pool, Figure 4).
//
// A workgroup owns 128 query rows of one (sequence, KV head): 128/G new tokens x the G
// query heads that read that KV head, so every K/V tile staged in LDS serves all heads
// of the group.  Four waves own 32 rows each.  The key loop walks the sequence's block
// table in 64-key tiles (four 16-token blocks):
//   * the whole workgroup loads the next tile from HBM into registers while the current
//     one is computed (coalesced 16-byte loads; a (block, head) tile is contiguous);
//   * K goes to LDS row-major (padded rows) as bf16; V goes to LDS transposed (dims x
//     keys) as fp16 (exact conversion), transposed in registers 4 keys x 8 dims at a
//     time; V rows past the sequence end are stored as zeros;
//   * S^T = K Q^T with v_mfma_f32_32x32x16_bf16: Q^T stays in registers for the whole
//     loop; in the C layout each lane holds one query row, so the online softmax needs
//     a single cross-lane step and the probabilities (rounded to fp16, which keeps 11
//     significant bits) feed O^T += V^T P^T (v_mfma_f32_32x32x16_f16) directly as the B
//     operand, in the same register order as the V^T fragments read from LDS.
// Workgroups of the same (sequence, KV head) are mapped onto one XCD so its L2 serves
// the shared prefix to all of them.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerWave = 32;
constexpr int kRows = 4 * kRowsPerWave;   // 128 query rows per workgroup
constexpr int kKT = 64;                   // keys per tile

template <int D>
struct PrefillSmem {
  static constexpr int kStride = D + 8;        // K rows (bf16): 16-byte pad
  static constexpr int vtStride = kKT + 8;     // V^T rows (bf16)
  uint16_t k[kKT * kStride];
  uint16_t vt[D * vtStride];
};

template <int D, int G>
__global__ __launch_bounds__(kThreads, 2) void gqa_prefill_kernel(GqaPrefillArgs a) {
  constexpr int KS = D / 16;          // QK k-steps (32x32x16)
  constexpr int MT = D / 32;          // O^T tiles of 32 dims
  constexpr int KCH = kKT * D / 8;    // 16-byte K chunks per tile
  constexpr int KPT = KCH / kThreads; // K chunks per thread
  constexpr int VGR = (kKT / 4) * (D / 8);  // (4 keys x 8 dims) V groups per tile
  constexpr int TT = kRows / G;       // new tokens per workgroup
  using Sm = PrefillSmem<D>;
  __shared__ __attribute__((aligned(16))) Sm sm;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int Hq = a.num_q_heads, Hkv = a.num_kv_heads;
  const int n_tiles = (a.max_new_len + TT - 1) / TT;
  const int logical = xcd_swizzle(blockIdx.x, gridDim.x);
  const int tile = logical % n_tiles;
  const int g = (logical / n_tiles) % Hkv;
  const int s = logical / (n_tiles * Hkv);
  const int nl = min(a.new_len[s], a.max_new_len);
  const int tok0 = tile * TT;
  if (tok0 >= nl) return;
  const int cached = a.cached_len[s];
  const int total = min(cached + nl, a.max_total_len);
  const int n_lblocks = (total + 15) >> 4;
  const int32_t* bt_row = a.bt + (size_t)s * a.bt_stride;
  const size_t head_stride = (size_t)16 * D;

  // ---- this lane's query row (B operand column / C column = lane % 32)
  const int c32 = lane & 31, h32 = lane >> 5;
  const int rr = wave * kRowsPerWave + c32;
  const int tok = tok0 + rr / G, hh = rr % G;
  const bool row_ok = tok < nl;
  const int tok_c = row_ok ? tok : nl - 1;
  const int pos = min(cached + tok_c, total - 1);
  const size_t q_row = (size_t)(a.q_start[s] + tok_c) * Hq + g * G + hh;
  u32x4 qb[KS];
  {
    const uint16_t* qp = a.q + q_row * D + 8 * h32;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qb[ks] = ld16(qp + 16 * ks);
  }
  // keys needed by this workgroup / this wave
  const int last_tok_wg = min(tok0 + TT, nl) - 1;
  const int kv_end = min(cached + last_tok_wg + 1, total);
  const int wave_min_pos = cached + min(tok0 + (wave * kRowsPerWave) / G, nl - 1);
  const int wave_max_pos = min(cached + min(tok0 + (wave * kRowsPerWave + kRowsPerWave - 1) / G, nl - 1), total - 1);

  f32x16 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[mt][i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  // ---- register prefetch of one K/V tile
  u32x4 kreg[KPT];
  u32x4 vreg[4];
  auto load_tile = [&](int kt) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int c = tid + kThreads * i;
      const int key = c / (D / 8), dc = c % (D / 8);
      const int pb = phys_block(bt_row, (kt + key) >> 4, n_lblocks, a.num_blocks);
      kreg[i] = pb >= 0 ? ld16(a.k + ((size_t)pb * Hkv + g) * head_stride + (size_t)(key & 15) * D + 8 * dc)
                        : u32x4{0, 0, 0, 0};
    }
    if (tid < VGR) {
      const int kg = tid % (kKT / 4), dc = tid / (kKT / 4);
      const int pb = phys_block(bt_row, (kt + 4 * kg) >> 4, n_lblocks, a.num_blocks);
      if (pb >= 0) {
        const uint16_t* vp = a.v + ((size_t)pb * Hkv + g) * head_stride + (size_t)((4 * kg) & 15) * D + 8 * dc;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          vreg[e] = (kt + 4 * kg + e < total) ? ld16(vp + (size_t)e * D) : u32x4{0, 0, 0, 0};
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) vreg[e] = u32x4{0, 0, 0, 0};
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int c = tid + kThreads * i;
      const int key = c / (D / 8), dc = c % (D / 8);
      st16(sm.k + key * Sm::kStride + 8 * dc, kreg[i]);
    }
    if (tid < VGR) {
      const int kg = tid % (kKT / 4), dc = tid / (kKT / 4);
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int w = 0; w < 4; ++w) vreg[e][w] = bf16x2_to_f16x2(vreg[e][w]);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        u32x2 lo, hi;
        lo.x = __builtin_amdgcn_perm(vreg[1][w], vreg[0][w], 0x05040100u);
        lo.y = __builtin_amdgcn_perm(vreg[3][w], vreg[2][w], 0x05040100u);
        hi.x = __builtin_amdgcn_perm(vreg[1][w], vreg[0][w], 0x07060302u);
        hi.y = __builtin_amdgcn_perm(vreg[3][w], vreg[2][w], 0x07060302u);
        *reinterpret_cast<u32x2*>(sm.vt + (8 * dc + 2 * w) * Sm::vtStride + 4 * kg) = lo;
        *reinterpret_cast<u32x2*>(sm.vt + (8 * dc + 2 * w + 1) * Sm::vtStride + 4 * kg) = hi;
      }
    }
  };

  load_tile(0);
  for (int kt = 0; kt < kv_end; kt += kKT) {
    __syncthreads();
    store_tile();
    __syncthreads();
    if (kt + kKT < kv_end) load_tile(kt + kKT);
    if (kt > wave_max_pos) continue;   // this wave's rows see none of these keys
    // ---- S^T = K Q^T, two 32-key sub-tiles
    f32x16 sacc[2];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[st][i] = 0.f;
      const uint16_t* kp = sm.k + (32 * st + c32) * Sm::kStride + 8 * h32;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        sacc[st] = mfma32x32x16(*reinterpret_cast<const u32x4*>(kp + 16 * ks), qb[ks], sacc[st]);
    }
    // ---- scale, causal mask, online softmax (log2 domain)
    const bool need_mask = kt + kKT - 1 > wave_min_pos;
    float mx = -INFINITY;
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float v = sacc[st][i] * a.scale_log2;
        if (need_mask) {
          const int key = kt + 32 * st + 8 * (i >> 2) + 4 * h32 + (i & 3);
          v = key <= pos ? v : -INFINITY;
        }
        sacc[st][i] = v;
        mx = fmaxf(mx, v);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    float alpha = 1.f, rs = 0.f;
    if (m_new != -INFINITY) {
      alpha = fast_exp2(m_run - m_new);
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = fast_exp2(sacc[st][i] - m_new);
          sacc[st][i] = p;
          rs += p;
        }
    } else {
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[st][i] = 0.f;
    }
    l_run = l_run * alpha + rs;
    m_run = m_new;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] *= alpha;
    // ---- O^T += V^T P^T, four 16-key k-steps
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int st = ks >> 1, r0 = 8 * (ks & 1);
      u32x4 pb;
      pb.x = pack_f16x2(sacc[st][r0 + 0], sacc[st][r0 + 1]);
      pb.y = pack_f16x2(sacc[st][r0 + 2], sacc[st][r0 + 3]);
      pb.z = pack_f16x2(sacc[st][r0 + 4], sacc[st][r0 + 5]);
      pb.w = pack_f16x2(sacc[st][r0 + 6], sacc[st][r0 + 7]);
      const int kbase = 32 * st + 16 * (ks & 1) + 4 * h32;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const uint16_t* vp = sm.vt + (32 * mt + c32) * Sm::vtStride + kbase;
        const u32x2 lo = *reinterpret_cast<const u32x2*>(vp);
        const u32x2 hi = *reinterpret_cast<const u32x2*>(vp + 8);
        acc[mt] = mfma32x32x16_f16(u32x4{lo.x, lo.y, hi.x, hi.y}, pb, acc[mt]);
      }
    }
  }

  // ---- normalise and write
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (!row_ok) return;
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  uint16_t* op = a.out + q_row * D;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      u32x2 w;
      w.x = pack_bf16x2(acc[mt][4 * q4 + 0] * inv, acc[mt][4 * q4 + 1] * inv);
      w.y = pack_bf16x2(acc[mt][4 * q4 + 2] * inv, acc[mt][4 * q4 + 3] * inv);
      *reinterpret_cast<u32x2*>(op + 32 * mt + 8 * q4 + 4 * h32) = w;
    }
  if (a.lse != nullptr && h32 == 0)
    a.lse[q_row] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
}

template <int D>
hipError_t launch_d(const GqaPrefillArgs& a, int G, unsigned grid, hipStream_t stream) {
  switch (G) {
    case 1: hipLaunchKernelGGL((gqa_prefill_kernel<D, 1>), dim3(grid), dim3(kThreads), 0, stream, a); break;
    case 2: hipLaunchKernelGGL((gqa_prefill_kernel<D, 2>), dim3(grid), dim3(kThreads), 0, stream, a); break;
    case 4: hipLaunchKernelGGL((gqa_prefill_kernel<D, 4>), dim3(grid), dim3(kThreads), 0, stream, a); break;
    case 8: hipLaunchKernelGGL((gqa_prefill_kernel<D, 8>), dim3(grid), dim3(kThreads), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gqa_prefill(const GqaPrefillArgs& a, hipStream_t stream) {
  const int G = a.num_q_heads / a.num_kv_heads;
  const int TT = kRows / G;
  const unsigned n_tiles = (unsigned)((a.max_new_len + TT - 1) / TT);
  const unsigned grid = n_tiles * a.num_kv_heads * a.num_seqs;
  if (grid == 0) return hipSuccess;
  return a.head_dim == 128 ? launch_d<128>(a, G, grid, stream) : launch_d<64>(a, G, grid, stream);
}

}  // namespace pa
