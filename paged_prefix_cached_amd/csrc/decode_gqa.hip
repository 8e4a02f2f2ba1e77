// Paged GQA decode (bf16 K/V, block size 16) that reads every distinct KV block once per
// group of sequences, with split-K over the context and a fixed-order combine.
//
// Sources: vLLM AgentX article (news.ainew.jp), "Re-evaluating agentic workloads" (>96 %
// prefix-cache hits; sub-agents fork from the parent context, so sequences in flight share
// long prefixes), "Hybrid KV cache management" (one shared block pool: shared prefixes are
// the same physical blocks, Figure 4) and "Kimi K3" (partial outputs and their
// log-sum-exp merged with online softmax, Figure 7).
//
// Work unit = (group of consecutive sequences, KV head g, split j).  A group holds
// M = 32 / (T*G) sequences, so its T query tokens x G heads per sequence fill the 32 rows
// of a v_mfma_f32_32x32x16 tile (cfg: 8 sequences x 4 heads).  For each 32-key tile of the
// split (two 16-token blocks) the wave looks up every member's pair of physical blocks and
// processes each DISTINCT pair once, for all member rows that reference it (ballot +
// readlane, no LDS): blocks shared by forked sequences are fetched from HBM once instead of
// once per sequence.  Correctness never depends on the grouping; a batch whose sessions
// are not adjacent just shares less.
//
// Per processed pair a wave:
//   * has issued the pair's K and V loads while the previous pair was being computed
//     (register double buffering: one pass always in flight per wave);
//   * uses K straight from registers as the A operand of S^T = K Q^T (lane l: key l%32);
//     Q^T fragments come from LDS, staged once per workgroup (B operand, lane = query row);
//   * masks rows that do not reference the pair and keys past each row's position, then
//     updates its online softmax in-lane (one xor-32 step per row);
//   * writes V (bf16; rows past the pair's longest member zeroed) row-major into its LDS
//     slice and accumulates O^T += V^T P^T with two v_mfma_f32_32x32x16_bf16, P split
//     into bf16 hi + lo parts (P keeps ~16 significant bits: rounding P to one bf16 would
//     cost ~1.5e-3 relative error in O); the V^T fragments come from
//     ds_read_b64_tr_b16 transpose reads, P straight from registers.
// The accumulator is rescaled only when a row's running maximum grows, which after the
// first tiles of a long context is rare.
// The 4 waves of a workgroup take tiles w, w+4, ... of the split; their states are merged
// pairwise through LDS in a fixed order, and the split's normalised partial output plus
// its log2-sum-exp go to the workspace.  combine_kernel merges splits in order.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kWaves = 4;
constexpr int kTile = 32;               // keys per pass (two 16-token blocks)

template <int D>
struct DecodeSmem {
  static constexpr int kVStride = D + 16;   // bf16 per V row: 32-byte pad, conflict-free tr reads
  static constexpr int kQStride = D + 8;    // bf16 per Q row: 16-byte pad
  uint16_t v[kWaves][kTile * kVStride];
  uint16_t q[32 * kQStride];
  int32_t bt[32][kDecodeSplitGqa / 16 + 1];  // the group's block ids for this split (-1: none)
};

__device__ __forceinline__ int members_per_group(int R) { return R >= 32 ? 1 : 32 / R; }

// One distinct (block pair) pass of a tile.
struct Pass {
  int kb, bA, bB, Lp;
  bool in;
};

template <int D>
__global__ __launch_bounds__(256, 2) void gqa_decode_kernel(GqaDecodeArgs a) {
  constexpr int KS = D / 16;   // QK k-steps (32x32x16)
  constexpr int MT = D / 32;   // O^T tiles of 32 dims
  constexpr int DC = D / 8;    // 16-byte chunks per V row
  constexpr int VG = D / 64;   // (4 keys x 8 dims) V groups per lane per pass
  using Sm = DecodeSmem<D>;
  __shared__ __attribute__((aligned(16))) Sm sm;
  __shared__ float mrg_ml[2][2][32];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int c32 = lane & 31, h32 = lane >> 5;
  const int Hq = a.num_q_heads, Hkv = a.num_kv_heads;
  const int G = Hq / Hkv, T = a.q_per_seq, R = T * G;
  const int M = members_per_group(R);
  const int n_groups = (a.num_seqs + M - 1) / M;
  const int units = n_groups * Hkv;
  const int split = blockIdx.x / units;
  const int grp = (blockIdx.x % units) / Hkv;
  const int g = blockIdx.x % Hkv;
  const int s0 = grp * M;

  // ---- this lane's query row: member m, token t, head hh
  const int m = c32 / R, rr = c32 % R;
  const int s = s0 + m;
  const bool row_ok = (m < M) && (s < a.num_seqs);
  const int L = row_ok ? min(a.context_len[s], a.max_context_len) : 0;
  const int t = rr / G, hh = rr % G;
  const int pos = L - T + t;                      // keys <= pos are visible
  int Lg = L;                                     // group-wide longest context
#pragma unroll
  for (int o = 16; o > 0; o >>= 1) Lg = max(Lg, __shfl_xor(Lg, o));
  const int k_begin = split * kDecodeSplitGqa;
  if (k_begin >= Lg) return;                      // uniform for the whole workgroup
  const int k_end = min(Lg, k_begin + kDecodeSplitGqa);
  const size_t head_stride = (size_t)16 * D;

  // ---- the group's block-table slice for this split -> LDS (validated ids, -1 = none),
  // so the pass loop never waits on a global load before issuing its K/V loads
  const int lb_base = k_begin >> 4;
  const int n_lb = ((k_end + 15) >> 4) - lb_base;
  for (int c = tid; c < M * n_lb; c += 256) {
    const int mm = c / n_lb, j = c % n_lb, sm_ = s0 + mm;
    int b = -1;
    if (sm_ < a.num_seqs) {
      const int Lm = min(a.context_len[sm_], a.max_context_len);
      b = phys_block(a.bt + (size_t)sm_ * a.bt_stride, lb_base + j, (Lm + 15) >> 4, a.num_blocks);
    }
    sm.bt[mm][j] = b;
  }
  // ---- Q of the group's 32 rows -> LDS once per workgroup (B operand of S^T = K Q^T)
  for (int c = tid; c < 32 * DC; c += 256) {
    const int r = c / DC, dc = c % DC;
    const int mr = r / R, rr2 = r % R, sr = s0 + mr;
    u32x4 v = {0, 0, 0, 0};
    if (mr < M && sr < a.num_seqs)
      v = ld16(a.q + ((size_t)(sr * T + rr2 / G) * Hq + g * G + rr2 % G) * D + 8 * dc);
    st16(sm.q + r * Sm::kQStride + 8 * dc, v);
  }
  __syncthreads();

  f32x16 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[mt][i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  uint16_t* vs = sm.v[wave];

  // rows of the group that reach past a tile need no zeroing of that tile's V rows
  int Lmin = row_ok ? L : 0x7fffffff;
#pragma unroll
  for (int o = 16; o > 0; o >>= 1) Lmin = min(Lmin, __shfl_xor(Lmin, o));

  // ---- pass iterator over this wave's tiles (kb = k_begin + 32 w, + 128, ...)
  int it_kb = k_begin + wave * kTile - kWaves * kTile;
  uint64_t it_todo = 0;
  int it_p0 = -1, it_p1 = -1;
  auto next_pass = [&](Pass& P) -> bool {
    while (it_todo == 0) {
      it_kb += kWaves * kTile;
      if (it_kb >= k_end) return false;
      const int j0 = (it_kb >> 4) - lb_base;
      it_p0 = row_ok ? sm.bt[m][j0] : -1;
      it_p1 = (row_ok && j0 + 1 < n_lb) ? sm.bt[m][j0 + 1] : -1;
      it_todo = __ballot((it_p0 >= 0 || it_p1 >= 0) && h32 == 0);
    }
    const int lead = __builtin_ctzll(it_todo);
    P.kb = it_kb;
    P.bA = __builtin_amdgcn_readlane(it_p0, lead);
    P.bB = __builtin_amdgcn_readlane(it_p1, lead);
    P.in = (it_p0 == P.bA) && (it_p1 == P.bB);
    it_todo &= ~__ballot(P.in && h32 == 0);
    if (it_kb + kTile <= Lmin) {
      P.Lp = 0x7fffffff;                          // interior tile: every key is valid data
    } else {                                      // longest context among the pass's rows
      int lp = P.in ? L : 0;
#pragma unroll
      for (int o = 16; o > 0; o >>= 1) lp = max(lp, __shfl_xor(lp, o));
      P.Lp = lp;
    }
    return true;
  };
  // K rows straight into the A operand (lane: key c32 of the pass); V as 4 keys x 8 dims.
  // Interior passes (both blocks present, no tail) take an unconditional path.
  auto issue = [&](const Pass& P, u32x4 (&kf)[KS], u32x4 (&vr)[VG][4]) {
    if (P.bA >= 0 && P.bB >= 0 && P.Lp == 0x7fffffff) {
      const int blk = c32 < 16 ? P.bA : P.bB;
      const uint16_t* kp = a.k + ((size_t)blk * Hkv + g) * head_stride + (size_t)(c32 & 15) * D + 8 * h32;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) kf[ks] = ld16(kp + 16 * ks);
#pragma unroll
      for (int j = 0; j < VG; ++j) {
        const int gi = lane + 64 * j, dc = gi % DC, kg = gi / DC;
        const int vb = kg < 4 ? P.bA : P.bB;
        const uint16_t* vp = a.v + ((size_t)vb * Hkv + g) * head_stride + (size_t)(4 * (kg & 3)) * D + 8 * dc;
#pragma unroll
        for (int e = 0; e < 4; ++e) vr[j][e] = ld16(vp + (size_t)e * D);
      }
      return;
    }
    const int blk = c32 < 16 ? P.bA : P.bB;
    if (blk >= 0) {
      const uint16_t* kp = a.k + ((size_t)blk * Hkv + g) * head_stride + (size_t)(c32 & 15) * D + 8 * h32;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) kf[ks] = ld16(kp + 16 * ks);
    } else {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) kf[ks] = u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int j = 0; j < VG; ++j) {
      const int gi = lane + 64 * j, dc = gi % DC, kg = gi / DC;
      const int vb = kg < 4 ? P.bA : P.bB;
      if (vb >= 0) {
        const uint16_t* vp = a.v + ((size_t)vb * Hkv + g) * head_stride + (size_t)(4 * (kg & 3)) * D + 8 * dc;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          vr[j][e] = (P.kb + 4 * kg + e < P.Lp) ? ld16(vp + (size_t)e * D) : u32x4{0, 0, 0, 0};
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) vr[j][e] = u32x4{0, 0, 0, 0};
      }
    }
  };
  const int m16 = lane & 15, gq = (lane >> 4) & 1;
  Pass nxt;
  u32x4 kfA[KS], kfB[KS], vr_n[VG][4];
  // One pass with its K in kf; the next pass is issued into kf_o (ping-pong) and vr_n.
  auto process = [&](u32x4 (&kf)[KS], u32x4 (&kf_o)[KS]) -> bool {
    const Pass cur = nxt;
    // ---- V (bf16) -> LDS row-major; frees the V registers for the next pass
#pragma unroll
    for (int j = 0; j < VG; ++j) {
      const int gi = lane + 64 * j, dc = gi % DC, kg = gi / DC;
#pragma unroll
      for (int e = 0; e < 4; ++e) st16(vs + (4 * kg + e) * Sm::kVStride + 8 * dc, vr_n[j][e]);
    }
    // the next pass's loads are in flight while this one is computed
    const bool more = next_pass(nxt);
    if (more) issue(nxt, kf_o, vr_n);
    // ---- S^T = K Q^T (Q^T fragments from LDS)
    const uint16_t* qp = sm.q + c32 * Sm::kQStride + 8 * h32;
    f32x16 sacc = mfma32x32x16(kf[0], *reinterpret_cast<const u32x4*>(qp), f32x16{});
#pragma unroll
    for (int ks = 1; ks < KS; ++ks)
      sacc = mfma32x32x16(kf[ks], *reinterpret_cast<const u32x4*>(qp + 16 * ks), sacc);
    // ---- mask + online softmax (log2 domain); lane = one row, 16 keys
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = cur.kb + 8 * (i >> 2) + 4 * h32 + (i & 3);
      const float v = (cur.in && key <= pos) ? sacc[i] * a.scale_log2 : -INFINITY;
      sacc[i] = v;
      mx = fmaxf(mx, v);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    // rescale only when some row's running max moved (exact: alpha = 1 otherwise)
    if (__ballot(m_new > m_run) != 0) {
      const float alpha = m_run == -INFINITY ? 0.f : fast_exp2(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[mt] *= alpha;
      m_run = m_new;
    }
    float rs = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float p = m_run == -INFINITY ? 0.f : fast_exp2(sacc[i] - m_run);
      sacc[i] = p;
      rs += p;
    }
    l_run += rs;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      // P = P_hi + P_lo, both bf16: the pair carries ~16 significant bits of P
      u32x4 ph, pl;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float a0 = sacc[8 * ks + 2 * w], a1 = sacc[8 * ks + 2 * w + 1];
        const uint32_t hv = pack_bf16x2(a0, a1);
        ph[w] = hv;
        pl[w] = pack_bf16x2(a0 - __uint_as_float(hv << 16), a1 - __uint_as_float(hv & 0xffff0000u));
      }
      // this lane's keys: kbase + 0..3 and kbase + 8..11 (the P^T register order)
      const int kbase = 16 * ks + 4 * h32;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const uint16_t* vp = vs + (kbase + (m16 >> 2)) * Sm::kVStride + 32 * mt + 16 * gq + 4 * (m16 & 3);
        const u32x2 lo = lds_read_tr16(vp);
        const u32x2 hi = lds_read_tr16(vp + 8 * Sm::kVStride);
        const u32x4 va = u32x4{lo.x, lo.y, hi.x, hi.y};
        acc[mt] = mfma32x32x16(va, ph, acc[mt]);
        acc[mt] = mfma32x32x16(va, pl, acc[mt]);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    return more;
  };
  bool have = next_pass(nxt);
  if (have) issue(nxt, kfA, vr_n);
  while (have) {
    have = process(kfA, kfB);
    if (!have) break;
    have = process(kfB, kfA);
  }

  // ---- merge the 4 wave states pairwise in a fixed order: (w0+w2) + (w1+w3)
  l_run += __shfl_xor(l_run, 32);
  float* buf = reinterpret_cast<float*>(&sm.v[0][0]);   // [2][32 rows][D] floats
  auto put = [&](int slot) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        *reinterpret_cast<f32x4*>(buf + ((size_t)slot * 32 + c32) * D + 32 * mt + 8 * q4 + 4 * h32) =
            f32x4{acc[mt][4 * q4], acc[mt][4 * q4 + 1], acc[mt][4 * q4 + 2], acc[mt][4 * q4 + 3]};
    if (h32 == 0) { mrg_ml[slot][0][c32] = m_run; mrg_ml[slot][1][c32] = l_run; }
  };
  auto take = [&](int slot) {
    const float mo = mrg_ml[slot][0][c32], lo = mrg_ml[slot][1][c32];
    const float Mx = fmaxf(m_run, mo);
    const float sa = (m_run == -INFINITY) ? 0.f : fast_exp2(m_run - Mx);
    const float sb = (mo == -INFINITY) ? 0.f : fast_exp2(mo - Mx);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x4 o = *reinterpret_cast<const f32x4*>(buf + ((size_t)slot * 32 + c32) * D + 32 * mt + 8 * q4 + 4 * h32);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[mt][4 * q4 + i] = acc[mt][4 * q4 + i] * sa + o[i] * sb;
      }
    l_run = l_run * sa + lo * sb;
    m_run = Mx;
  };
  __syncthreads();
  if (wave >= 2) put(wave - 2);
  __syncthreads();
  if (wave < 2) take(wave);
  __syncthreads();
  if (wave == 1) put(0);
  __syncthreads();
  if (wave != 0) return;
  take(0);
  if (!row_ok) return;
  const int TR = T * Hq;
  const size_t pidx = ((size_t)s * a.max_splits + split) * TR + (size_t)t * Hq + g * G + hh;
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
  float* op = a.part_o + pidx * D;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4)
      *reinterpret_cast<f32x4*>(op + 32 * mt + 8 * q4 + 4 * h32) =
          f32x4{acc[mt][4 * q4] * inv, acc[mt][4 * q4 + 1] * inv, acc[mt][4 * q4 + 2] * inv, acc[mt][4 * q4 + 3] * inv};
  if (h32 == 0) a.part_lse[pidx] = l_run > 0.f ? m_run + __log2f(l_run) : -INFINITY;
}

}  // namespace

hipError_t launch_gqa_decode(const GqaDecodeArgs& a, hipStream_t stream) {
  const int R = a.q_per_seq * (a.num_q_heads / a.num_kv_heads);
  const int M = R >= 32 ? 1 : 32 / R;
  const unsigned n_groups = (unsigned)((a.num_seqs + M - 1) / M);
  const unsigned grid = (unsigned)a.max_splits * n_groups * a.num_kv_heads;
  if (grid == 0) return hipSuccess;
  if (a.head_dim == 128)
    hipLaunchKernelGGL((gqa_decode_kernel<128>), dim3(grid), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((gqa_decode_kernel<64>), dim3(grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------
// Fixed-order combine of split partials: for each (sequence, row) with n splits,
//   M = max_j lse_j,  o = sum_j 2^(lse_j - M) o_j / sum_j 2^(lse_j - M),
// summed for j = 0 .. n-1 in order, so results are identical run to run.
namespace {
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  const int row = blockIdx.x % a.rows, s = blockIdx.x / a.rows;
  const int L = min(a.context_len[s], a.max_context_len);
  const int n = L > 0 ? (L + a.split - 1) / a.split : 0;
  const size_t stride = (size_t)a.rows;
  const float* lse_p = a.part_lse + (size_t)s * a.max_splits * stride + row;
  float M = -INFINITY;
  for (int j = 0; j < n; ++j) M = fmaxf(M, lse_p[j * stride]);
  float den = 0.f;
  for (int j = 0; j < n; ++j) {
    const float lj = lse_p[j * stride];
    den += (M == -INFINITY || lj == -INFINITY) ? 0.f : fast_exp2(lj - M);
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
  const float* o_p = a.part_o + ((size_t)s * a.max_splits * stride + row) * a.head_dim;
  uint16_t* out = a.out + ((size_t)s * a.rows + row) * a.head_dim;
  for (int d = threadIdx.x; d < a.head_dim; d += blockDim.x) {
    float num = 0.f;
    for (int j = 0; j < n; ++j) {
      const float lj = lse_p[j * stride];
      const float w = (M == -INFINITY || lj == -INFINITY) ? 0.f : fast_exp2(lj - M);
      num += w * o_p[(size_t)j * stride * a.head_dim + d];
    }
    out[d] = __builtin_bit_cast(uint16_t, (__bf16)(num * inv));
  }
  if (a.lse != nullptr && threadIdx.x == 0)
    a.lse[(size_t)s * a.rows + row] = den > 0.f ? (M + __log2f(den)) * kLn2 : -INFINITY;
}
}  // namespace

hipError_t launch_combine(const CombineArgs& a, hipStream_t stream) {
  const unsigned grid = (unsigned)a.num_seqs * a.rows;
  if (grid == 0) return hipSuccess;
  const int threads = a.head_dim >= 256 ? 256 : a.head_dim;
  hipLaunchKernelGGL(combine_kernel, dim3(grid), dim3(threads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pa
