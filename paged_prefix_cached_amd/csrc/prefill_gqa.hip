// Prefix-cached suffix prefill over a paged bf16 pool (GQA / MHA, block size 16).
//
// Sources: vLLM AgentX article (news.ainew.jp), "Re-evaluating agentic workloads" (each
// turn re-sends the history; most of it is a cached prefix, the new prefill is short)
// and "Hybrid KV cache management" (one shared block pool, Figure 4).
//
// A workgroup owns 256 query rows of one (sequence, KV head): 256/G new tokens x the G
// query heads that read that KV head, so every K/V tile staged in LDS serves all heads
// of the group.  Eight waves own 32 rows each (two per SIMD; the 148 KB of LDS for two
// tile buffers leave one workgroup per CU): a tile fetched from HBM serves twice the
// rows of a four-wave workgroup.  The key loop walks the sequence's block table in
// 128-key tiles (eight 16-token blocks), one barrier per tile:
//   * at the top of step t, tile t+1 (loaded into registers during step t-1, coalesced
//     16-byte loads of contiguous (block, head) tiles) is stored into the other LDS
//     buffer -- K row-major as bf16, V row-major as fp16 (exact conversion), V rows past
//     the sequence end as zeros -- and tile t+2's loads go out;
//   * S^T = K Q^T with v_mfma_f32_32x32x16_bf16: Q^T stays in registers for the whole
//     loop; in the C layout each lane holds one query row, so the online softmax needs a
//     single cross-lane step.  The softmax scale is fused into the exponent
//     (p = 2^(s c - m), max taken on raw scores), and the reference maximum moves only
//     when a row's maximum grows by more than 2^8 (log2 units): probabilities up to 256
//     stay exact enough in fp16, and the accumulator is almost never rescaled;
//   * O^T += V^T P^T with v_mfma_f32_32x32x16_f16: P (fp16, 11 significant bits) comes
//     straight from registers, V^T fragments from ds_read_b64_tr_b16 transpose reads of
//     the row-major V tile (the reduction index relabelled to match the C layout).
// Row strides: K 272 B (68 dwords: the 16 rows of a b128 read phase hit distinct banks),
// V (D + 32) fp16 (D/2 + 16 dwords, 16 or 48 mod 64: the 4 rows of a transpose read
// phase hit distinct banks).
// Workgroups of the same (sequence, KV head) are mapped onto one XCD so its L2 serves
// the shared prefix to all of them; the XCDs take different KV heads.  Without a split,
// the latest tiles are dealt first (under the causal mask they see the most keys).
// Split-K (prefill_split_len): when the tiles alone cannot fill the GPU and the contexts
// are long, each workgroup takes one key range of its tile and writes fp32 partials
// (o, log2-sum-exp) that the decode combine kernel merges in range order.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

#ifndef PA_PREFILL_WAVES
#define PA_PREFILL_WAVES 8
#endif
constexpr int kWaves = PA_PREFILL_WAVES;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsPerWave = 32;
constexpr int kRows = kWaves * kRowsPerWave;   // query rows per workgroup
#ifndef PA_PREFILL_KT
#define PA_PREFILL_KT 128
#endif
constexpr int kKT = PA_PREFILL_KT;        // keys per tile
constexpr int kST = kKT / 32;             // 32-key sub-tiles per tile

template <int D>
struct PrefillSmem {
  static constexpr int kStride = D + 8;        // K rows (bf16)
  static constexpr int vStride = D + 32;       // V rows (fp16)
  uint16_t k[2][kKT * kStride];
  uint16_t v[2][kKT * vStride];
};

template <int D, int G>
__global__ __launch_bounds__(kThreads, 2) void gqa_prefill_kernel(GqaPrefillArgs a) {
  constexpr int KS = D / 16;          // QK k-steps (32x32x16)
  constexpr int MT = D / 32;          // O^T tiles of 32 dims
  constexpr int KCH = kKT * D / 8;    // 16-byte chunks per K (or V) tile
  constexpr int KPT = KCH / kThreads; // chunks per thread
  constexpr int TT = kRows / G;       // new tokens per workgroup
  using Sm = PrefillSmem<D>;
  static_assert(KCH % kThreads == 0, "whole chunks per thread");
  __shared__ __attribute__((aligned(16))) Sm sm;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int Hq = a.num_q_heads, Hkv = a.num_kv_heads;
  const int n_tiles = (a.max_new_len + TT - 1) / TT;
  const int n_split = a.split_len > 0 ? a.max_splits : 1;
  const int logical = xcd_swizzle(blockIdx.x, gridDim.x);
  // tiles of one (sequence, key range) run together on one XCD (shared K/V in its L2);
  // the KV head varies slowest, so the XCDs split the work by head and a long sequence
  // is spread over all of them
  // unsplit, a later tile sees more keys (causal): the longest tiles are dealt first
  const int tile = a.split_len > 0 ? logical % n_tiles : n_tiles - 1 - logical % n_tiles;
  const int split = (logical / n_tiles) % n_split;
  const int s = (logical / (n_tiles * n_split)) % a.num_seqs;
  const int g = logical / (n_tiles * n_split * a.num_seqs);
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
  int kv_end = min(cached + last_tok_wg + 1, total);
  // split-K: this workgroup's key range [kv_begin, kv_end)
  const int kv_begin = a.split_len > 0 ? split * a.split_len : 0;
  if (a.split_len > 0) kv_end = min(kv_end, kv_begin + a.split_len);
  if (kv_begin >= kv_end) return;                      // no row of the tile sees this range
  const int wave_min_pos = cached + min(tok0 + (wave * kRowsPerWave) / G, nl - 1);
  const int wave_max_pos = min(cached + min(tok0 + (wave * kRowsPerWave + kRowsPerWave - 1) / G, nl - 1), total - 1);
  const float c = a.scale_log2;

  f32x16 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[mt][i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;   // m_run in scaled log2 units

  // ---- register prefetch of one K/V tile: chunk ci = tid + kThreads i holds 8 dims of one key.
  // A wave's 64 lanes cover 64/(D/8) consecutive keys of one 16-token block, so chunk i of a
  // wave lies in a block known from the wave index alone: each wave looks up only its own
  // KPT block ids (scalar loads, same address in every lane) and reads K and V through one
  // buffer resource per (block, KV head): a scalar base plus a loop-invariant lane offset.
  // The loads go out together once the ids are back, so a tile costs one table round trip
  // (vector-memory counters complete in order).  A block past the sequence or out of range
  // gets zero records (its loads return zeros); V rows past the sequence end (last tile
  // only) are read at an offset past the records.
  constexpr int kKeysPerRound = kThreads / (D / 8);     // keys covered by one round of chunks
  constexpr int kKeysPerWave = 64 / (D / 8);            // keys of one wave in one round
  static_assert(16 % kKeysPerWave == 0 && kKeysPerRound % 16 == 0, "a wave's chunk stays in one block");
  const int wave_key0 = __builtin_amdgcn_readfirstlane(wave) * kKeysPerWave;
  const int lane_off = (((tid / (D / 8)) & 15) * D + 8 * (tid % (D / 8))) * 2;   // bytes
  u32x4 kreg[KPT], vreg[KPT];
  int pbs[KPT];
  // Branch-free: the entry is read at min(lb, n_lblocks - 1) (n_lblocks >= 1 here) and
  // discarded past the end, so the KPT scalar loads share one wait.
  auto lookup_blocks = [&](int kt) {
    int raw[KPT];
#pragma unroll
    for (int i = 0; i < KPT; ++i)
      raw[i] = bt_row[min((kt + wave_key0 + kKeysPerRound * i) >> 4, n_lblocks - 1)];
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int lb = (kt + wave_key0 + kKeysPerRound * i) >> 4;
      pbs[i] = (lb < n_lblocks && raw[i] >= 0 && raw[i] < a.num_blocks) ? raw[i] : -1;
    }
  };
  auto load_kv = [&](int kt) {
    const bool tail = kt + kKT > total;                // uniform: the tile holds the end
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int pb = pbs[i];
      const size_t blk = ((size_t)(pb >= 0 ? pb : 0) * Hkv + g) * head_stride;
      const __amdgpu_buffer_rsrc_t rk =
          __builtin_amdgcn_make_buffer_rsrc((void*)(a.k + blk), (short)0, pb >= 0 ? 32 * D : 0, 0x00020000);
      const __amdgpu_buffer_rsrc_t rv =
          __builtin_amdgcn_make_buffer_rsrc((void*)(a.v + blk), (short)0, pb >= 0 ? 32 * D : 0, 0x00020000);
      const int key = tid / (D / 8) + kKeysPerRound * i;
      kreg[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, lane_off, 0, 0));
      const int voff = (tail && kt + key >= total) ? (int)0x80000000 : lane_off;
      vreg[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, voff, 0, 0));
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int ci = tid + kThreads * i;
      const int key = ci / (D / 8), dc = ci % (D / 8);
      st16(sm.k[buf] + key * Sm::kStride + 8 * dc, kreg[i]);
      const u32x4 v16 = {bf16x2_to_f16x2(vreg[i].x), bf16x2_to_f16x2(vreg[i].y),
                         bf16x2_to_f16x2(vreg[i].z), bf16x2_to_f16x2(vreg[i].w)};
      st16(sm.v[buf] + key * Sm::vStride + 8 * dc, v16);
    }
  };

  // V^T fragment offsets (fp16 units): first read rows 16 kk + 4 h + n/4 of a 32-key
  // sub-tile, dims 32 mt + 16 (g16 & 1) + 4 (n & 3); second read 8 rows further.
  const int g16 = lane >> 4, n16 = lane & 15;
  const int v_lo = (4 * h32 + (n16 >> 2)) * Sm::vStride + 16 * (g16 & 1) + 4 * (n16 & 3);

  auto compute = [&](int buf, int kt) {
    const uint16_t* kt_s = sm.k[buf];
    const uint16_t* vt_s = sm.v[buf];
    // ---- S^T = K Q^T, 32-key sub-tiles
    // k-step outer, sub-tile inner: consecutive MFMAs accumulate into different tiles and
    // each k-step's K reads have the previous k-step's kST MFMAs to land behind
    f32x16 sacc[kST];
#pragma unroll
    for (int st = 0; st < kST; ++st)
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[st][i] = 0.f;
    const uint16_t* kp = kt_s + c32 * Sm::kStride + 8 * h32;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int st = 0; st < kST; ++st)
        sacc[st] = mfma32x32x16(*reinterpret_cast<const u32x4*>(kp + 32 * st * Sm::kStride + 16 * ks), qb[ks], sacc[st]);
    // ---- causal mask (diagonal tiles only) and the row maximum on raw scores
    float mx = -INFINITY;
    if (kt + kKT - 1 > wave_min_pos) {
      // register i of sub-tile st holds key kt + 32 st + 4 h32 + 8 (i/4) + i%4
#pragma unroll
      for (int st = 0; st < kST; ++st) {
        const int lim = pos - kt - 32 * st - 4 * h32;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          if (8 * (i >> 2) + (i & 3) > lim) sacc[st][i] = -INFINITY;
          mx = fmaxf(mx, sacc[st][i]);
        }
      }
    } else {                                     // every key of the tile is visible
#pragma unroll
      for (int st = 0; st < kST; ++st)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[st][i]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32)) * c;
    if (__ballot(mx > m_run + 8.f) != 0) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = m_run == -INFINITY ? 0.f : fast_exp2(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[mt] *= alpha;
      m_run = m_new;
    }
    const float neg_m = m_run == -INFINITY ? 0.f : -m_run;   // fully masked rows: p = 0
    float rs = 0.f;
#pragma unroll
    for (int st = 0; st < kST; ++st)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = fast_exp2(fmaf(sacc[st][i], c, neg_m));
        sacc[st][i] = p;
        rs += p;
      }
    l_run += rs;
    // ---- O^T += V^T P^T: k-step (st, kk) holds keys 32 st + 16 kk + 8 (j/4) + 4 h + j%4
#pragma unroll
    for (int st = 0; st < kST; ++st)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int r0 = 8 * kk;
        const u32x4 pb = {pack_f16x2(sacc[st][r0 + 0], sacc[st][r0 + 1]), pack_f16x2(sacc[st][r0 + 2], sacc[st][r0 + 3]),
                          pack_f16x2(sacc[st][r0 + 4], sacc[st][r0 + 5]), pack_f16x2(sacc[st][r0 + 6], sacc[st][r0 + 7])};
        const uint16_t* vp = vt_s + (32 * st + 16 * kk) * Sm::vStride + v_lo;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const u32x2 lo = lds_read_tr16(vp + 32 * mt);
          const u32x2 hi = lds_read_tr16(vp + 8 * Sm::vStride + 32 * mt);
          acc[mt] = mfma32x32x16_f16(u32x4{lo.x, lo.y, hi.x, hi.y}, pb, acc[mt]);
        }
      }
  };

  // ---- pipeline: one barrier per tile; buffer t&1 holds tile t
  lookup_blocks(kv_begin);
  load_kv(kv_begin);
  store_tile(0);
  if (kv_begin + kKT < kv_end) {
    lookup_blocks(kv_begin + kKT);
    load_kv(kv_begin + kKT);
  }
  __syncthreads();
  for (int kt = kv_begin, t = 0; kt < kv_end; kt += kKT, ++t) {
    const int buf = t & 1;
    if (kt + kKT < kv_end) {
      const bool more = kt + 2 * kKT < kv_end;
      if (more) lookup_blocks(kt + 2 * kKT);     // in flight while tile t+1 is stored
      store_tile(buf ^ 1);                       // tile t+1, read last in step t-1
      if (more) load_kv(kt + 2 * kKT);
    }
    if (kt <= wave_max_pos) compute(buf, kt);    // else this wave's rows see none of these keys
    __syncthreads();
  }

  // ---- normalise and write
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (!row_ok) return;
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (a.split_len > 0) {
    // partial of this key range: o (normalised over the range) and its log2-sum-exp, at
    // [s * max_new_len + token][split][head] -- indexed by the sequence's own token slot,
    // never by q_start, so the workspace of num_seqs * max_new_len token slots always holds it
    const size_t slot = (((size_t)s * a.max_new_len + tok_c) * a.max_splits + split) * Hq + g * G + hh;
    float* po = a.part_o + slot * D;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        *reinterpret_cast<f32x4*>(po + 32 * mt + 8 * q4 + 4 * h32) =
            f32x4{acc[mt][4 * q4] * inv, acc[mt][4 * q4 + 1] * inv, acc[mt][4 * q4 + 2] * inv, acc[mt][4 * q4 + 3] * inv};
    if (h32 == 0) a.part_lse[slot] = l_tot > 0.f ? m_run + __log2f(l_tot) : -INFINITY;
    return;
  }
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

// Split-K when the unsplit grid would leave the compute units short of work and the key
// ranges are long: 8,192-key ranges (a workgroup then handles at most 64 key tiles;
// measured on the chunked step: 4,096 / 8,192 / 16,384 / 32,768 -> 1.26 / 1.23 / 1.29 / 1.26 ms).
#ifndef PA_PREFILL_SPLIT_LEN
#define PA_PREFILL_SPLIT_LEN 8192
#endif
constexpr int kPrefillSplitLen = PA_PREFILL_SPLIT_LEN;
int prefill_split_len(int num_seqs, int num_q_heads, int num_kv_heads, int max_new_len, int max_total_len) {
  if (num_seqs <= 0 || num_kv_heads <= 0 || max_new_len <= 0) return 0;
  const int cus = device_cus();
  const int G = num_q_heads / num_kv_heads;
  const int TT = kRows / (G > 0 ? G : 1);
  const long wgs = (long)((max_new_len + TT - 1) / TT) * num_kv_heads * num_seqs;
  if (wgs >= 4L * cus || max_total_len <= 2 * kPrefillSplitLen) return 0;
  return kPrefillSplitLen;
}

hipError_t launch_gqa_prefill(const GqaPrefillArgs& a, hipStream_t stream) {
  const int G = a.num_q_heads / a.num_kv_heads;
  const int TT = kRows / G;
  const unsigned n_tiles = (unsigned)((a.max_new_len + TT - 1) / TT);
  const unsigned n_split = a.split_len > 0 ? (unsigned)a.max_splits : 1u;
  const unsigned grid = n_tiles * n_split * a.num_kv_heads * a.num_seqs;
  if (grid == 0) return hipSuccess;
  return a.head_dim == 128 ? launch_d<128>(a, G, grid, stream) : launch_d<64>(a, G, grid, stream);
}

}  // namespace pa
