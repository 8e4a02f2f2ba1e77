// Indexer scores: I[i,t] = scale_t * sum_h w[i,h] * max(0, <q[i,h,:], e4m3(k_t)>) for
// t <= pos(i), else -inf -- or, with the MXFP4 keys of the packed per-block layout (vLLM
// AgentX article, "Hybrid KV cache management": the FP4 indexer), the same sum over the
// decoded keys (E2M1 elements times their E8M0 group scale).
//
// Sources: vLLM AgentX article (news.ainew.jp), "DeepSeek V4" (the indexer has 64 heads
// but yields one global top-k per token); GLM-5.3 report (aisoku.org), "What's new" (the
// indexer picks 2,048 tokens; its cost is quadratic in the prompt).  The per-token key
// scale is positive, so it commutes with the ReLU and is applied once after the head sum.
//
// A workgroup of 8 waves owns 8 query rows (one per wave) and a chunk of keys.  Key
// tiles of 64 tokens (one block each; the block id is read a tile ahead) are gathered
// through the block table and staged in LDS once for all 8 queries (two buffers; the
// following tile's bytes are in registers meanwhile).  Each wave keeps its query's 64 heads
// in registers (A operand) and computes C[heads x keys] per 16-key sub-tile; in the C
// layout a lane holds 4 heads of one key, so the weighted ReLU head sum is 16 fused
// multiply-adds in registers (ReLU as one v_med3_f32) plus a 2-step reduction across the 4
// lane groups (row swaps).  The four 16-key sub-tiles of a tile form one basic block, their
// score stores after it, so one sub-tile's MFMAs overlap the previous one's head sums.
//   FP8 keys: the tile stays E4M3 in LDS (144-byte rows) and feeds
//     v_mfma_f32_16x16x128_f8f6f4 as read; each head's bf16 query row is scaled by 2^qs_h
//     and split into two E4M3 terms (exact for elements at least 2^-9 of the head's
//     largest), so a head tile takes two MFMAs (hi, lo), and 2^-qs_h is folded into w_h
//     (ReLU commutes with a positive factor).
//   MXFP4 keys: the tile is upcast to bf16 in LDS (272-byte rows) and the bf16 queries feed
//     v_mfma_f32_16x16x32_bf16, four k-steps per head tile.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kD = 128, kBs = 64;
#ifndef PA_INDEXER_WAVES
#define PA_INDEXER_WAVES 8
#endif
constexpr int kWaves = PA_INDEXER_WAVES;
constexpr int kThreads = 64 * kWaves;
constexpr int kKT = 64;                  // keys per LDS tile
constexpr int kChunk = 8192;             // keys per workgroup
constexpr int kKStride = kD + 8;         // bf16 per key row in LDS (272 B), MXFP4 keys
constexpr int kKStride8 = kD + 16;       // bytes per key row in LDS (144 B), FP8 keys: the
                                         // 16 rows of a sub-tile start in distinct banks

__device__ __forceinline__ int find_seq(const int32_t* q_start, int num_seqs, int i) {
  int lo = 0, hi = num_seqs - 1;
  while (lo < hi) {                      // last s with q_start[s] <= i
    const int mid = (lo + hi + 1) >> 1;
    if (q_start[mid] <= i) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// FP4 (MXFP4 keys of the packed layout): a key row is 64 bytes, element 2j in the low
// nibble of byte j, with one E8M0 scale code per 32 elements; the upcast to bf16 applies
// the group scale (2^(e-127), built as the float with exponent field e), exact for codes
// in [2, 252].  Keys carry no per-token scale (1 in the score).
template <int NHT, bool FP4>   // head tiles of 16 (num_heads / 16)
__global__ __launch_bounds__(kThreads) void indexer_kernel(IndexerArgs a) {
  constexpr int kRowB = FP4 ? 2 * kKStride : kKStride8;   // LDS bytes per key row
  __shared__ __attribute__((aligned(16))) uint8_t k_s[2][kKT * kRowB];
  __shared__ float sc_s[2][kKT];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int m16 = lane & 15, grp = lane >> 4;
  const int n_chunks = (a.max_total_len + kChunk - 1) / kChunk;
  const int qblk = blockIdx.x / n_chunks, chunk = blockIdx.x % n_chunks;
  const int i0 = qblk * kWaves;
  const int s = find_seq(a.q_start, a.num_seqs, i0);
  // every row of the block must belong to sequence s: rows of another sequence are
  // handled by a second pass over the same block (rare: only at sequence boundaries)
  const int c0 = chunk * kChunk;
  for (int seq = s; seq < a.num_seqs; ++seq) {
    const int qs = a.q_start[seq];
    const int nl = min(a.new_len[seq], a.max_new_len);
    if (qs > i0 + kWaves - 1) break;
    const int cached = a.cached_len[seq];
    const int total = min(cached + nl, a.max_total_len);
    const int n_lblocks = (total + kBs - 1) / kBs;
    const int32_t* bt_row = a.bt + (size_t)seq * a.bt_stride;
    const int i = i0 + wave;
    const bool mine = i < a.n_q && i >= qs && i < qs + nl;
    const int pos = mine ? min(cached + (i - qs), total - 1) : -1;
    // highest position of the block's rows in this sequence
    const int i_last = min(i0 + kWaves, min(qs + nl, a.n_q)) - 1;
    const int blk_max_pos = min(cached + (i_last - qs), total - 1);
    const int c1 = min(c0 + kChunk, a.max_total_len);
    if (mine && chunk == 0) a.valid_len[i] = pos + 1;
    // ---- Q in registers, A operand.  MXFP4 keys: [16 heads x 32 dims] bf16 per (head
    // tile, k-step).  FP8 keys: [16 heads x 128 dims] as two E4M3 terms per head tile, lane
    // group grp holding dims 32 grp .. + 31 (the same byte order as the key operand).
    u32x4 qa[FP4 ? NHT : 1][4];
    i32x8 qhi[FP4 ? 1 : NHT], qlo[FP4 ? 1 : NHT];
    float wv[NHT][4];
    if (mine) {
      const uint16_t* qp = a.q_idx + (size_t)i * (NHT * 16) * kD;
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht) {
#pragma unroll
        for (int r = 0; r < 4; ++r) wv[ht][r] = a.w[(size_t)i * (NHT * 16) + 16 * ht + 4 * grp + r];
        if constexpr (FP4) {
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) qa[ht][ks] = ld16(qp + (size_t)(16 * ht + m16) * kD + 32 * ks + 8 * grp);
        } else {
          u32x4 v[4];
          uint32_t amax = 0u;
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            v[c] = ld16(qp + (size_t)(16 * ht + m16) * kD + 32 * grp + 8 * c);
            amax = bf16x8_absmax_bits(v[c], amax);
          }
          // the head's largest over its four lane groups (lanes l, l ^ 16, l ^ 32, l ^ 48)
          const auto r16 = __builtin_amdgcn_permlane16_swap(amax, amax, false, false);
          amax = max(r16[0], r16[1]);
          const auto r32 = __builtin_amdgcn_permlane32_swap(amax, amax, false, false);
          const int qs = split_scale_exp(max(r32[0], r32[1]));
          const float up = exp2i(qs);
          uint32_t hw[8], lw[8];
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            bf16x4_split_e4m3(v[c].x, v[c].y, up, hw[2 * c], lw[2 * c]);
            bf16x4_split_e4m3(v[c].z, v[c].w, up, hw[2 * c + 1], lw[2 * c + 1]);
          }
          qhi[ht] = as_i32x8(u32x4{hw[0], hw[1], hw[2], hw[3]}, u32x4{hw[4], hw[5], hw[6], hw[7]});
          qlo[ht] = as_i32x8(u32x4{lw[0], lw[1], lw[2], lw[3]}, u32x4{lw[4], lw[5], lw[6], lw[7]});
          // C row 4 grp + r of this head tile is head 16 ht + 4 grp + r, whose qs lane 4 grp + r holds
#pragma unroll
          for (int r = 0; r < 4; ++r) wv[ht][r] *= exp2i(-__shfl(qs, 4 * grp + r));
        }
      }
    } else {
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht) {
        if constexpr (FP4) {
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) qa[ht][ks] = u32x4{0, 0, 0, 0};
        } else {
          qhi[ht] = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
          qlo[ht] = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) wv[ht][r] = 0.f;
      }
    }
    float* srow = mine ? a.scores + (size_t)i * a.score_stride : nullptr;
    const int kc_end = min(c1, blk_max_pos + 1);
    // Tile pipeline, one barrier per tile: at the top of step t the FP8 bytes of tile t+1
    // (loaded during step t-1) are upcast into LDS buffer (t+1)&1, which the barrier
    // ending step t-1 freed; tile t+2's loads go out; tile t is computed from buffer t&1.
    // 64 keys x 128 B = 512 chunks of 16 B; chunk tid + kThreads j of a thread holds key
    // (tid + kThreads j) / 8, bytes 16 (tid % 8) ..
    constexpr int CPT = kKT * (kD / 16) / kThreads;
    static_assert(CPT * kThreads == kKT * (kD / 16), "whole chunks per thread");
    const int key = tid >> 3, dc = tid & 7;   // dims 16 dc .. 16 dc + 15 of key `key`
    u32x4 raw[CPT];                           // FP8: 16 codes; FP4: 16 codes in .x, .y
    float rsc[CPT];                           // FP8: the key's scale; FP4: the group scale
    // A 64-key tile is exactly one 64-token block.  Its table entry is read one tile ahead
    // of its key loads (a vector load from an opaque copy of the index, so it is counted
    // with the key loads, in order, and never waits alone): the key loads of a tile never
    // wait for a table round trip.  Entries past the end are read clamped and discarded.
    auto bt_raw = [&](int kb) -> int {
      int lb = min(kb / kBs, n_lblocks - 1);
      asm volatile("" : "+v"(lb));
      return bt_row[lb];
    };
    auto bt_ok = [&](int kb, int raw_id) -> int {
      return (kb / kBs < n_lblocks && raw_id >= 0 && raw_id < a.num_blocks) ? raw_id : -1;
    };
    auto load_tile = [&](int kb, int pb) {
#pragma unroll
      for (int j = 0; j < CPT; ++j) {
        const int t = kb + key + (kThreads / 8) * j;
        const bool ok = pb >= 0 && t < total;
        const size_t blk = (size_t)(ok ? pb : 0);
        if constexpr (FP4) {
          const u32x2 c = ok ? *reinterpret_cast<const u32x2*>(a.keys + blk * a.blk_bytes + (t % kBs) * (kD / 2) + 8 * dc)
                             : u32x2{0, 0};
          raw[j] = u32x4{c.x, c.y, 0, 0};
          const uint32_t e = ok ? a.key_sbase[blk * a.sblk_bytes + (t % kBs) * 4 + (dc >> 1)] : 127u;
          rsc[j] = __uint_as_float(e << 23);
        } else {
          raw[j] = ok ? ld16(a.keys + blk * a.blk_bytes + (t % kBs) * kD + 16 * dc) : u32x4{0, 0, 0, 0};
          if (dc == 0)
            rsc[j] = ok ? *reinterpret_cast<const float*>(a.key_sbase + blk * a.sblk_bytes + (t % kBs) * 4) : 0.f;
        }
      }
    };
    auto store_tile = [&](int buf) {
#pragma unroll
      for (int j = 0; j < CPT; ++j) {
        const int kj = key + (kThreads / 8) * j;
        if constexpr (FP4) {
          // byte b of each word: elements 2b (low nibble) and 2b + 1
          uint32_t bf[8];
          const uint32_t wx = raw[j].x, wy = raw[j].y;
          const float sc = rsc[j];
          bf[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wx, sc, 0));
          bf[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wx, sc, 1));
          bf[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wx, sc, 2));
          bf[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wx, sc, 3));
          bf[4] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wy, sc, 0));
          bf[5] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wy, sc, 1));
          bf[6] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wy, sc, 2));
          bf[7] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wy, sc, 3));
          uint8_t* kp = k_s[buf] + kj * kRowB + 32 * dc;
          st16(kp, u32x4{bf[0], bf[1], bf[2], bf[3]});
          st16(kp + 16, u32x4{bf[4], bf[5], bf[6], bf[7]});
        } else {
          st16(k_s[buf] + kj * kRowB + 16 * dc, raw[j]);    // E4M3 bytes as loaded
        }
        if (dc == 0) sc_s[buf][kj] = FP4 ? 1.f : rsc[j];
      }
    };
    int id_next = -1;                                // raw table entry of tile tt+2
    if (c0 < kc_end) {                               // (then n_lblocks >= 1)
      __syncthreads();                               // a previous sequence pass is done with LDS
      load_tile(c0, bt_ok(c0, bt_raw(c0)));
      store_tile(0);
      if (c0 + kKT < kc_end) load_tile(c0 + kKT, bt_ok(c0 + kKT, bt_raw(c0 + kKT)));
      id_next = bt_raw(c0 + 2 * kKT);
      __syncthreads();
    }
    for (int kb = c0, tt = 0; kb < kc_end; kb += kKT, ++tt) {
      const int buf = tt & 1;
      if (kb + kKT < kc_end) {
        store_tile(buf ^ 1);                         // tile tt+1 (its loads went out last step)
        if (kb + 2 * kKT < kc_end) {
          const int pb = bt_ok(kb + 2 * kKT, id_next);
          load_tile(kb + 2 * kKT, pb);
          id_next = bt_raw(kb + 3 * kKT);
        }
      }
      if (mine && kb <= pos) {
        // all four 16-key sub-tiles in one basic block (the stores come after), so one
        // sub-tile's MFMAs overlap the previous one's ReLU sums
        float part[kKT / 16];
#pragma unroll
        for (int st = 0; st < kKT / 16; ++st) {
          float acc = 0.f;
          if constexpr (FP4) {
            u32x4 kb4[4];
            const uint8_t* kp = k_s[buf] + (16 * st + m16) * kRowB + 16 * grp;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) kb4[ks] = *reinterpret_cast<const u32x4*>(kp + 64 * ks);
#pragma unroll
            for (int ht = 0; ht < NHT; ++ht) {
              f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
              for (int ks = 0; ks < 4; ++ks) c = mfma16x16x32(qa[ht][ks], kb4[ks], c);
#pragma unroll
              for (int r = 0; r < 4; ++r) acc = fmaf(wv[ht][r], __builtin_amdgcn_fmed3f(c[r], 0.f, 3.402823466e38f), acc);   // ReLU (finite scores)
            }
          } else {
            // key 16 st + m16, dims 32 grp .. + 31
            const uint8_t* kp = k_s[buf] + (16 * st + m16) * kRowB + 32 * grp;
            const i32x8 kb = as_i32x8(*reinterpret_cast<const u32x4*>(kp), *reinterpret_cast<const u32x4*>(kp + 16));
#pragma unroll
            for (int ht = 0; ht < NHT; ++ht) {
              f32x4 c = {0.f, 0.f, 0.f, 0.f};
              c = mfma16x16x128_fp8(qhi[ht], kb, c);
              c = mfma16x16x128_fp8(qlo[ht], kb, c);
#pragma unroll
              for (int r = 0; r < 4; ++r) acc = fmaf(wv[ht][r], __builtin_amdgcn_fmed3f(c[r], 0.f, 3.402823466e38f), acc);   // ReLU (finite scores)
            }
          }
          // sum over the 4 lane groups (lanes l, l^16, l^32, l^48 hold the same key) with
          // row swaps: every lane adds the same two operands, so all copies agree
          const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(acc), __float_as_uint(acc), false, false);
          const float a16 = __uint_as_float(r16[0]) + __uint_as_float(r16[1]);
          const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(a16), __float_as_uint(a16), false, false);
          part[st] = __uint_as_float(r32[0]) + __uint_as_float(r32[1]);
        }
#pragma unroll
        for (int st = 0; st < kKT / 16; ++st) {
          const int t = kb + 16 * st + m16;
          if (grp == 0 && t <= pos && t < c1) srow[t] = part[st] * sc_s[buf][16 * st + m16] + 0.f;
        }
      }
      __syncthreads();
    }
    // keys of this chunk past the row's position: -inf (the tile loop wrote t <= pos)
    if (mine) {
      for (int t = max(c0, pos + 1) + lane; t < c1; t += 64) srow[t] = -INFINITY;
    }
  }
}

template <bool FP4>
hipError_t launch_h(const IndexerArgs& a, unsigned grid, hipStream_t stream) {
  switch (a.num_heads / 16) {
    case 1: hipLaunchKernelGGL((indexer_kernel<1, FP4>), dim3(grid), dim3(kThreads), 0, stream, a); break;
    case 2: hipLaunchKernelGGL((indexer_kernel<2, FP4>), dim3(grid), dim3(kThreads), 0, stream, a); break;
    case 3: hipLaunchKernelGGL((indexer_kernel<3, FP4>), dim3(grid), dim3(kThreads), 0, stream, a); break;
    case 4: hipLaunchKernelGGL((indexer_kernel<4, FP4>), dim3(grid), dim3(kThreads), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_indexer_scores(const IndexerArgs& a, hipStream_t stream) {
  const int n_chunks = (a.max_total_len + kChunk - 1) / kChunk;
  const unsigned grid = (unsigned)((a.n_q + kWaves - 1) / kWaves) * n_chunks;
  if (grid == 0) return hipSuccess;
  return a.fp4 ? launch_h<true>(a, grid, stream) : launch_h<false>(a, grid, stream);
}

}  // namespace pa
