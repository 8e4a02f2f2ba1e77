// Paged GQA decode (bf16 K/V, block size 16): split-K over the context with a
// fixed-order combine of the partial (output, log-sum-exp) pairs.
//
// Sources: vLLM AgentX article (news.ainew.jp), "Hybrid KV cache management" (one shared
// block pool, the page is the allocation unit, Figure 4) and "Kimi K3" (partial outputs
// and their log-sum-exp merged with online softmax, Figure 7).
//
// Work unit = (sequence s, KV head g, split j): the T*G query rows that read KV head g
// (T query tokens x G heads of the group) against keys [j*SPLIT, (j+1)*SPLIT).  A unit is
// one workgroup of 4 waves; wave w takes 32-key tiles w, w+4, w+8, ... of the split and
// keeps its own online-softmax state; the 4 states are merged through LDS and written
// as one normalised partial output plus its log2-sum-exp.
//
// Per 32-key tile (two 16-token blocks) a wave:
//   * loads each K block straight from HBM into the B operand of S = Q K^T (lane l reads
//     token l%16, 16 contiguous bytes per k-step: a 4 KB block is one coalesced sweep);
//   * computes S with v_mfma_f32_16x16x32_bf16 (Q rows r at MFMA row 4r when T*G <= 4,
//     so every lane holds a real score in register 0);
//   * updates the running max / sum with 16-lane reductions and exp2;
//   * writes V^T (dims x keys, fp16: exact conversion) into its LDS slice -- V arrives
//     4 tokens x 8 dims per lane and is transposed in registers; rows past the context
//     are zeros -- and P (fp16) into LDS, then accumulates O^T += V^T P^T with
//     v_mfma_f32_16x16x32_f16.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kWaves = 4;
constexpr int kTile = 32;               // keys per wave iteration
constexpr int kVtStride = kTile + 8;    // bf16 elements per V^T row (80 B: conflict-free)
constexpr int kPStride = kTile + 8;

template <int D, int NREG>
__global__ __launch_bounds__(256) void gqa_decode_kernel(GqaDecodeArgs a) {
  constexpr int KS = D / 32;   // QK k-steps
  constexpr int MT = D / 16;   // PV output tiles (16 dims each)
  constexpr int VG = D / 64;   // (4 keys x 8 dims) V groups per lane per tile
  __shared__ __attribute__((aligned(16))) uint16_t vt_s[kWaves * D * kVtStride];
  __shared__ __attribute__((aligned(16))) uint16_t p_s[kWaves * 16 * kPStride];
  __shared__ float mrg_ml[kWaves][2][16];

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int Hq = a.num_q_heads, Hkv = a.num_kv_heads;
  const int G = Hq / Hkv, T = a.q_per_seq, R = T * G;
  const int units = a.num_seqs * Hkv;
  const int split = blockIdx.x / units;
  const int s = (blockIdx.x % units) / Hkv;
  const int g = blockIdx.x % Hkv;
  const int L = min(a.context_len[s], a.max_context_len);
  const int k_begin = split * kDecodeSplitGqa;
  if (k_begin >= L) return;                       // uniform for the whole workgroup
  const int k_end = min(L, k_begin + kDecodeSplitGqa);
  const int n_lblocks = (L + 15) >> 4;
  const int32_t* bt_row = a.bt + (size_t)s * a.bt_stride;
  const size_t head_stride = (size_t)16 * D;      // one (block, head) tile

  // ---- Q as the A operand of S = Q K^T
  const int m16 = lane & 15, grp = lane >> 4;
  int qr = (NREG == 1) ? ((m16 & 3) == 0 ? (m16 >> 2) : -1) : m16;
  if (qr >= R) qr = -1;
  u32x4 qa[KS];
  if (qr >= 0) {
    const uint16_t* qp = a.q + ((size_t)(s * T + qr / G) * Hq + g * G + qr % G) * D + 8 * grp;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qa[ks] = ld16(qp + 32 * ks);
  } else {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qa[ks] = u32x4{0, 0, 0, 0};
  }

  // Rows held by this lane in the S tile (register i): MFMA row 4*grp + i.
  int srow[NREG], spos[NREG];
#pragma unroll
  for (int i = 0; i < NREG; ++i) {
    srow[i] = (NREG == 1) ? grp : 4 * grp + i;
    spos[i] = (srow[i] < R) ? (L - T + srow[i] / G) : -1;
  }
  float m_run[NREG], l_run[NREG];
#pragma unroll
  for (int i = 0; i < NREG; ++i) { m_run[i] = -INFINITY; l_run[i] = 0.f; }
  f32x4 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  uint16_t* vt = vt_s + wave * D * kVtStride;
  uint16_t* ps = p_s + wave * 16 * kPStride;
  const int ocol = lane & 15;                        // O^T column = query row

  for (int kb = k_begin + wave * kTile; kb < k_end; kb += kWaves * kTile) {
    const int lb0 = kb >> 4;
    // ---- issue all global loads of the tile
    u32x4 kf[2][KS];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const int pb = phys_block(bt_row, lb0 + st, n_lblocks, a.num_blocks);
      if (pb >= 0) {
        const uint16_t* kp = a.k + ((size_t)pb * Hkv + g) * head_stride + (size_t)m16 * D + 8 * grp;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) kf[st][ks] = ld16(kp + 32 * ks);
      } else {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) kf[st][ks] = u32x4{0, 0, 0, 0};
      }
    }
    u32x4 vr[VG][4];
#pragma unroll
    for (int j = 0; j < VG; ++j) {
      const int gi = lane + 64 * j, kg = gi & 7, dc = gi >> 3;
      const int pb = phys_block(bt_row, lb0 + (kg >> 2), n_lblocks, a.num_blocks);
      if (pb >= 0) {
        const uint16_t* vp = a.v + ((size_t)pb * Hkv + g) * head_stride + (size_t)(4 * (kg & 3)) * D + 8 * dc;
#pragma unroll
        for (int e = 0; e < 4; ++e) vr[j][e] = (kb + 4 * kg + e < L) ? ld16(vp + (size_t)e * D) : u32x4{0, 0, 0, 0};
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) vr[j][e] = u32x4{0, 0, 0, 0};
      }
    }
    // ---- S = Q K^T for the two 16-key sub-tiles
    f32x4 sacc[2];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      sacc[st] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) sacc[st] = mfma16x16x32(qa[ks], kf[st][ks], sacc[st]);
    }
    // ---- online softmax (log2 domain); P -> LDS as fp16 [row][key]
    float alpha[NREG];
#pragma unroll
    for (int i = 0; i < NREG; ++i) {
      const int k0 = kb + m16, k1 = kb + 16 + m16;
      float v0 = (k0 <= spos[i]) ? sacc[0][i] * a.scale_log2 : -INFINITY;
      float v1 = (k1 <= spos[i]) ? sacc[1][i] * a.scale_log2 : -INFINITY;
      float mx = wave_max_xor(fmaxf(v0, v1), 16);
      const float m_new = fmaxf(m_run[i], mx);
      float p0 = 0.f, p1 = 0.f;
      alpha[i] = 1.f;
      if (m_new != -INFINITY) {
        alpha[i] = fast_exp2(m_run[i] - m_new);
        p0 = fast_exp2(v0 - m_new);
        p1 = fast_exp2(v1 - m_new);
      }
      l_run[i] = l_run[i] * alpha[i] + p0 + p1;
      m_run[i] = m_new;
      if (srow[i] < R) {
        ps[srow[i] * kPStride + m16] = __builtin_bit_cast(uint16_t, (_Float16)p0);
        ps[srow[i] * kPStride + 16 + m16] = __builtin_bit_cast(uint16_t, (_Float16)p1);
      }
    }
    // ---- V^T -> LDS: transpose (4 keys x 8 dims) per group in registers
#pragma unroll
    for (int j = 0; j < VG; ++j) {
      const int gi = lane + 64 * j, kg = gi & 7, dc = gi >> 3;
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int w = 0; w < 4; ++w) vr[j][e][w] = bf16x2_to_f16x2(vr[j][e][w]);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        u32x2 lo, hi;
        lo.x = __builtin_amdgcn_perm(vr[j][1][w], vr[j][0][w], 0x05040100u);
        lo.y = __builtin_amdgcn_perm(vr[j][3][w], vr[j][2][w], 0x05040100u);
        hi.x = __builtin_amdgcn_perm(vr[j][1][w], vr[j][0][w], 0x07060302u);
        hi.y = __builtin_amdgcn_perm(vr[j][3][w], vr[j][2][w], 0x07060302u);
        *reinterpret_cast<u32x2*>(vt + (8 * dc + 2 * w) * kVtStride + 4 * kg) = lo;
        *reinterpret_cast<u32x2*>(vt + (8 * dc + 2 * w + 1) * kVtStride + 4 * kg) = hi;
      }
    }
    // ---- rescale O^T columns by their row's alpha (row c lives in lane group c/4 of S)
    float a_col;
    if (NREG == 1) {
      a_col = __shfl(alpha[0], 16 * (ocol < 4 ? ocol : 0));
    } else {
      float c0 = __shfl(alpha[0], 16 * (ocol >> 2));
      float c1 = __shfl(alpha[NREG > 1 ? 1 : 0], 16 * (ocol >> 2));
      float c2 = __shfl(alpha[NREG > 2 ? 2 : 0], 16 * (ocol >> 2));
      float c3 = __shfl(alpha[NREG > 3 ? 3 : 0], 16 * (ocol >> 2));
      const int q4 = ocol & 3;
      a_col = q4 == 0 ? c0 : (q4 == 1 ? c1 : (q4 == 2 ? c2 : c3));
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] *= a_col;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // ---- O^T += V^T P^T
    u32x4 pb = u32x4{0, 0, 0, 0};
    if (ocol < R) pb = *reinterpret_cast<const u32x4*>(ps + ocol * kPStride + 8 * grp);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const u32x4 va = *reinterpret_cast<const u32x4*>(vt + (m16 + 16 * mt) * kVtStride + 8 * grp);
      acc[mt] = mfma16x16x32_f16(va, pb, acc[mt]);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  // ---- merge the 4 wave states through LDS (reusing the V^T area)
#pragma unroll
  for (int i = 0; i < NREG; ++i) l_run[i] = wave_sum_xor(l_run[i], 16);
  __syncthreads();
  float* mrg_o = reinterpret_cast<float*>(vt_s);     // [kWaves][16][D] floats
  if (m16 == 0) {
#pragma unroll
    for (int i = 0; i < NREG; ++i) {
      if (srow[i] < 16) {
        mrg_ml[wave][0][srow[i]] = m_run[i];
        mrg_ml[wave][1][srow[i]] = l_run[i];
      }
    }
  }
  if (ocol < R) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) mrg_o[(wave * 16 + ocol) * D + 16 * mt + 4 * grp + i] = acc[mt][i];
  }
  __syncthreads();
  const int TR = T * Hq;
  const size_t part_base = ((size_t)s * a.max_splits + split) * TR;
  for (int idx = threadIdx.x; idx < R * D; idx += 256) {
    const int row = idx / D, d = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, mrg_ml[w][0][row]);
    float num = 0.f, den = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float mw = mrg_ml[w][0][row];
        const float sc = (mw == -INFINITY) ? 0.f : fast_exp2(mw - M);
        num += sc * mrg_o[(w * 16 + row) * D + d];
        den += sc * mrg_ml[w][1][row];
      }
    }
    const int rg = (row / G) * Hq + g * G + row % G;
    a.part_o[(part_base + rg) * D + d] = den > 0.f ? num / den : 0.f;
    if (d == 0) a.part_lse[part_base + rg] = den > 0.f ? M + __log2f(den) : -INFINITY;
  }
}

}  // namespace

hipError_t launch_gqa_decode(const GqaDecodeArgs& a, hipStream_t stream) {
  const int G = a.num_q_heads / a.num_kv_heads;
  const int R = a.q_per_seq * G;
  const unsigned grid = (unsigned)a.max_splits * a.num_seqs * a.num_kv_heads;
  if (grid == 0) return hipSuccess;
  if (a.head_dim == 128) {
    if (R <= 4) hipLaunchKernelGGL((gqa_decode_kernel<128, 1>), dim3(grid), dim3(256), 0, stream, a);
    else hipLaunchKernelGGL((gqa_decode_kernel<128, 4>), dim3(grid), dim3(256), 0, stream, a);
  } else {
    if (R <= 4) hipLaunchKernelGGL((gqa_decode_kernel<64, 1>), dim3(grid), dim3(256), 0, stream, a);
    else hipLaunchKernelGGL((gqa_decode_kernel<64, 4>), dim3(grid), dim3(256), 0, stream, a);
  }
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
