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
// Each head's bf16 query row is scaled by 2^qs_h and split into two E4M3 terms (exact for
// elements at least 2^-9 of the head's largest), so a head tile takes two FP8 MFMAs (hi,
// lo) per 16 keys, and 2^-qs_h is folded into w_h (ReLU commutes with a positive factor).
// The key tile stays in its stored format in LDS and is fed to the MFMA as read:
//   FP8 keys: E4M3 rows (144 bytes apart), v_mfma_f32_16x16x128_f8f6f4;
//   MXFP4 keys: E2M1 rows (80 bytes apart) and each row's four E8M0 codes,
//     v_mfma_scale_f32_16x16x128_f8f6f4 with the key operand in FP4 and, per lane, the
//     code of the 32-element group the lane holds as its scale (the MX block of the
//     instruction is the lane's 32 elements, which is one group of the key).
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
// LDS bytes per key row: the 16 rows of a sub-tile start in distinct banks
constexpr int kRowFp8 = kD + 16;         // FP8 keys: 128 bytes + 16
constexpr int kRowFp4 = kD / 2 + 16;     // MXFP4 keys: 64 bytes + 16

__device__ __forceinline__ int find_seq(const int32_t* q_start, int num_seqs, int i) {
  int lo = 0, hi = num_seqs - 1;
  while (lo < hi) {                      // last s with q_start[s] <= i
    const int mid = (lo + hi + 1) >> 1;
    if (q_start[mid] <= i) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// FP4 (MXFP4 keys of the packed layout): a key row is 64 bytes, element 2j in the low
// nibble of byte j, with one E8M0 scale code per 32 elements, applied by the MFMA; keys
// carry no per-token scale (1 in the score).
// Four waves per SIMD (two workgroups per CU): the compiler keeps a wave within 128 VGPRs,
// spilling a few loop-invariant values for 64 heads, and the second workgroup's waves hide
// the first's LDS and head-sum latencies (6.9 vs 7.9 ms at 4,096 x 135K, 64 heads).
template <int NHT, bool FP4>   // head tiles of 16 (num_heads / 16)
__global__ __launch_bounds__(kThreads, 4) void indexer_kernel(IndexerArgs a) {
  constexpr int kRowB = FP4 ? kRowFp4 : kRowFp8;
  __shared__ __attribute__((aligned(16))) uint8_t k_s[2][kKT * kRowB];
  __shared__ uint8_t e_s[2][FP4 ? kKT * 4 : 4];                 // MXFP4: key r's codes at 4 r
  __shared__ float sc_s[2][kKT];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: the row's values stay scalar
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
    // ---- Q in registers, A operand: [16 heads x 128 dims] as two E4M3 terms per head
    // tile.  The reduction index of an E4M3 operand's lane group grp is 16 grp + j for bytes
    // j < 16 and 64 + 16 grp + j - 16 for the rest, in both operands; an E2M1 operand's lane
    // group holds 32 grp .. + 31 in nibble order (measured).  FP8 keys: both operands take
    // dims 32 grp .. + 31 in byte order (the same layout, so the pairing is the identity).
    // MXFP4 keys: the key lane holds dims 32 grp .. + 31, so the query lane holds dims
    // 16 grp .. + 15 in bytes 0-15 and 64 + 16 grp .. + 15 in bytes 16-31.
    i32x8 qhi[NHT], qlo[NHT];
    float wv[NHT][4];
    if (mine) {
      const uint16_t* qp = a.q_idx + (size_t)i * (NHT * 16) * kD;
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht) {
        u32x4 v[4];
        uint32_t amax = 0u;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int d0 = FP4 ? (c < 2 ? 16 * grp + 8 * c : 64 + 16 * grp + 8 * (c - 2)) : 32 * grp + 8 * c;
          v[c] = ld16(qp + (size_t)(16 * ht + m16) * kD + d0);
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
        for (int r = 0; r < 4; ++r)
          wv[ht][r] = a.w[(size_t)i * (NHT * 16) + 16 * ht + 4 * grp + r] * exp2i(-__shfl(qs, 4 * grp + r));
      }
    } else {
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht) {
        qhi[ht] = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
        qlo[ht] = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
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
    float rsc[CPT];                           // FP8: the key's scale
    uint32_t rcode[CPT];                      // FP4: the E8M0 code of the thread's group
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
          rcode[j] = ok ? a.key_sbase[blk * a.sblk_bytes + (t % kBs) * 4 + (dc >> 1)] : 127u;
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
          *reinterpret_cast<u32x2*>(k_s[buf] + kj * kRowB + 8 * dc) = u32x2{raw[j].x, raw[j].y};
          if ((dc & 1) == 0) e_s[buf][4 * kj + (dc >> 1)] = (uint8_t)rcode[j];
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
            // key 16 st + m16, elements 32 grp .. + 31 (16 bytes) and their group's code
            const int kr = 16 * st + m16;
            const u32x4 k4 = *reinterpret_cast<const u32x4*>(k_s[buf] + kr * kRowB + 16 * grp);
            const int code = e_s[buf][4 * kr + grp];
            const i32x8 kb = as_i32x8(k4, u32x4{0, 0, 0, 0});
#pragma unroll
            for (int ht = 0; ht < NHT; ++ht) {
              f32x4 c = {0.f, 0.f, 0.f, 0.f};
              c = mfma16x16x128_fp8_fp4(qhi[ht], kb, code, c);
              c = mfma16x16x128_fp8_fp4(qlo[ht], kb, code, c);
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
