// MLA attention over the FP8 latent cache with the FP8 operands read straight from the
// gathered tile: paged decode (with MTP query tokens) and sparse MLA over indexer-selected
// tokens.
//
// Sources: vLLM AgentX article (news.ainew.jp), "Kimi K3" (MLA keeps one latent head;
// partial outputs merged by log-sum-exp) and "DeepSeek V4" (sparse MLA gathers the top-k
// KV entries, then attends); GLM-5.3 report (aisoku.org), "What's new" (the latent KV is
// shared by all 64 heads), its table (FP8 KV, MTP3) and "How to try" (prompts inside the
// top-k use the same sparse MQA kernel).
//
// MQA with d_qk = 576 (512 latent + 64 rope) and d_v = 512 (the latent itself).  Each wave
// owns 32 query rows outright: their Q (all 576 dims, two E4M3 terms) in registers and their output
// accumulator (32 rows x 512 dims fp32) in the 256 accumulation registers, one wave per
// SIMD.  No partial score is ever exchanged between waves; the NW waves of a workgroup
// (NW x 32 rows) share each 32-key tile.
//
// Keys go in 32-key tiles through an NBUF-deep LDS-DMA pipeline (global_load_lds, 16 bytes
// a lane, no registers held while the loads fly): tile t + NBUF - 1 is gathered while tile
// t is computed -- its row loads spread over the Q.K pass rather than issued in one burst --
// with one barrier per tile.  The tile stays FP8 in LDS, chunk-major: 16-byte
// chunk c of key r sits at c * 512 + 16 (r ^ 4 (c & 1)).  So a DMA lane fetches the same
// key for every chunk pair it loads (one row address per lane and tile), the Q.K fragment
// reads of a k-step cover 512 contiguous bytes, and the transposed V reads of a half-wave
// hit 64 distinct banks.  Per tile a wave computes
//   S^T = K Q^T with v_mfma_f32_32x32x64_f8f6f4 on the key bytes as they are: lane (key
//     r = lane % 32, half h = lane / 32) reads chunks 4 ks + 2 h and 4 ks + 2 h + 1 of its
//     key (dims 64 ks + 32 h .. + 31) with two ds_read_b128 per k-step, and the query row,
//     scaled by a power of two and split into two E4M3 terms, goes in as two MFMAs per
//     k-step, its fragments in the same byte order;
//   the softmax per row (lane = row, 16 keys; one lane-half swap per reduction), the
//     per-token scale folded into the scores (s * scale_t) and into P (p * scale_t);
//   O^T += V^T P^T: the V^T fragment (dim = lane % 32, 8 keys) is one ds_read_b64_tr_b8 --
//     within each group of 16 lanes, lane i receives byte i % 8 of the 8-byte reads of lanes
//     2k + i / 8 (k = 0..7) -- converted to fp16; the keys it covers are relabelled to match
//     the P fragment the lane already holds.
// LDS reads run ahead of their use (Q.K: kPre / 4 k-steps; V^T: kPre fragments).  Keys that are not to be read
// (unselected, past the range, bad block id) are fetched from a row of zeros: zero K, V and
// scale, and their scores are masked to -inf.
//
// The accumulator is written only by the MFMAs (any other write to it inside the loop makes
// the compiler move it out of the accumulation registers).  So the softmax keeps, per row,
// a reference maximum fixed at its first valid tile; probabilities stay <= 2^kSlack unless
// a later maximum passes the reference by more than kSlack.  A workgroup that sees that
// marks its output, and the exact two-stage kernel (mla_exact.hip) recomputes exactly those
// work units right after, in the same launch sequence.
#include <type_traits>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kDqk = 576, kDv = 512, kBs = 64;
constexpr int kKT = 32;                      // keys per tile
constexpr int kColB = kKT * 16;              // one chunk column: 32 keys x 16 bytes
constexpr int kTileB = kKT * kDqk;           // 18,432 bytes per tile
constexpr int kTileLoads = kTileB / 1024;    // 18 wave-loads of 1 KB (two chunk columns each)
constexpr int kQS = kDqk / 64;               // 9 Q.K k-steps of 64 dims (FP8 MFMA)
constexpr int kMT = kDv / 32;                // 16 output tiles of 32 dims
constexpr int kSelLds = 2048;                // sparse selections staged in LDS
constexpr uint32_t kNoRow = 0xffffff;        // staged row (24 bits) of an unread selection
constexpr float kSlack = 8.f;                // log2 units: probabilities stay <= 2^8
constexpr int kPre = 8;                      // LDS fragment reads in flight ahead of use

// Source of the DMA for keys that are not to be read (a latent row and a scale of zeros) and
// of the filler loads that keep every wave's DMA count equal: 1 KB of zeros.
__device__ __attribute__((aligned(16))) uint8_t kZeroRow[1024] = {};

// Eight FP8 (E4M3) bytes -> eight fp16 (exact), as an MFMA operand.
__device__ __forceinline__ u32x4 fp8x8_to_f16x8(u32x2 b) {
  const u32x2 lo = fp8x4_to_f16x4(b.x), hi = fp8x4_to_f16x4(b.y);
  return u32x4{lo.x, lo.y, hi.x, hi.y};
}

typedef __attribute__((address_space(3))) const uint8_t lds_u8;

__device__ __forceinline__ u32x4 lds_read_b128(lds_u8* base, int off) {
  return *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(base + off);
}

__device__ __forceinline__ u32x2 lds_read_tr8(lds_u8* base, int off) {
  typedef int i32x2 __attribute__((ext_vector_type(2)));
  auto* lp = (__attribute__((address_space(3))) i32x2*)(base + off);
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr8_b64_v2i32(lp));
}

// Wait until at most N vector-memory operations of this wave are outstanding (gfx9
// s_waitcnt encoding: vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
  asm volatile("" ::: "memory");
}
// The same for a wave-uniform count n in [0, N] (a chain of scalar branches).
template <int N>
__device__ __forceinline__ void wait_vm_upto(int n) {
  if (n >= N) wait_vm<N>();
  else if constexpr (N > 0) wait_vm_upto<N - 1>(n);
}

// NW waves (NW x 32 query rows) per workgroup, one wave per SIMD; NBUF tile buffers.
// STAGED (sparse): the selections' physical rows (k <= 2048, rows below 2^24 - 1) are staged
// in LDS once, 3 bytes each (6 KB: two workgroups of 4 tile buffers then fit on a CU);
// otherwise each tile resolves them from global memory.
template <bool SPARSE, int NW, int NBUF, bool STAGED>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(1, 1))) void mla_kernel(MlaDecodeArgs da,
                                                                                                   SparseMlaArgs sa) {
  static_assert(NBUF >= 2, "tile buffers");
  constexpr int NT = NW * 64;
  constexpr int RW = 32 * NW;                                 // query rows per workgroup
  // DMA wave-loads per tile: wave w issues loads w, w + NW, ...; the tile's scales go out
  // with the last wave's loads.
  constexpr int kLoadsMax = (kTileLoads + NW - 1) / NW;
  __shared__ __attribute__((aligned(16))) uint8_t raw[NBUF][kTileB];
  __shared__ __attribute__((aligned(16))) float tsc[NBUF][kKT];     // per-key scale (0 if invalid)
  __shared__ uint32_t tmask[NBUF];                                  // bit k: key k is valid
  __shared__ int32_t ovf_s[NW];                                     // per wave: a row overflowed
  constexpr bool kFiller = NW * kLoadsMax != kTileLoads;           // some waves have a spare load
  __shared__ __attribute__((aligned(16))) uint8_t spare[kFiller ? 1024 : 16];  // its target
  __shared__ int32_t bt_s[SPARSE ? 1 : kDecodeSplitMla / kBs + 1];
  __shared__ uint16_t sel_lo[SPARSE && STAGED ? kSelLds : 1];     // staged rows: bits 0-15
  __shared__ uint8_t sel_hi[SPARSE && STAGED ? kSelLds : 1];      // and bits 16-23

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Any use of the accumulation registers makes the compiler select the MFMA forms that
  // accumulate there: the 32 x 512 fp32 output tile lives in them and the query fragments
  // and everything else in the ordinary registers.
  asm volatile("; accumulators in the accumulation registers" ::: "a0");
  const int l32 = lane & 31, h = lane >> 5;

  // ---- work unit
  const uint16_t* qbase;
  const int32_t* bt_row;
  const int32_t* sel_g = nullptr;
  const uint8_t* kv;
  const uint8_t* ksb;
  int64_t blk_bytes, sblk_bytes;
  int Hq, n_keys, k_begin = 0, n_lblocks, L = 0, T = 1, row0, unit = 0, unit_split = 0;
  int lb_base = 0, n_bt = 0, num_blocks;
  float scale_log2;
  if constexpr (SPARSE) {
    Hq = sa.num_q_heads;
    const int rblocks = (Hq + RW - 1) / RW;
    // consecutive query tokens select overlapping keys: keep them on one XCD (shared L2)
    const int bid = xcd_swizzle(blockIdx.x, gridDim.x);
    const int i = bid / rblocks;
    row0 = (bid % rblocks) * RW;
    unit = i;
    qbase = sa.q + (size_t)i * Hq * kDqk;
    kv = sa.kv; ksb = sa.kv_sbase; num_blocks = sa.num_blocks;
    blk_bytes = sa.blk_bytes; sblk_bytes = sa.sblk_bytes;
    bt_row = sa.bt + (size_t)sa.q_seq[i] * sa.bt_stride;
    sel_g = sa.topk + (size_t)i * sa.k;
    n_keys = sa.k;
    n_lblocks = sa.bt_stride;
    scale_log2 = sa.scale_log2;
  } else {
    Hq = da.num_q_heads;
    T = da.q_per_seq;
    const int rows = T * Hq;
    const int rblocks = (rows + RW - 1) / RW;
    const int n_units = da.num_seqs * da.max_splits * rblocks;
    // (sequence, split) units go to the XCDs round robin, with each sequence's split order
    // rotated by its index: every XCD gets about 1/8 of every sequence's keys
    const int logical = xcd_unit_swizzle(blockIdx.x, n_units, rblocks);
    const int rb = logical % rblocks;
    unit = logical / (rblocks * da.max_splits);
    unit_split = ((logical / rblocks) % da.max_splits + unit) % da.max_splits;
    row0 = rb * RW;
    L = min(da.context_len[unit], da.max_context_len);
    k_begin = unit_split * kDecodeSplitMla;
    if (k_begin >= L) return;                         // uniform for the workgroup
    n_keys = min(L - k_begin, kDecodeSplitMla);
    qbase = da.q + (size_t)unit * rows * kDqk;
    kv = da.kv; ksb = da.kv_sbase; num_blocks = da.num_blocks;
    blk_bytes = da.blk_bytes; sblk_bytes = da.sblk_bytes;
    bt_row = da.bt + (size_t)unit * da.bt_stride;
    n_lblocks = (L + kBs - 1) / kBs;
    lb_base = k_begin / kBs;
    n_bt = (k_begin + n_keys + kBs - 1) / kBs - lb_base;
    scale_log2 = da.scale_log2;
  }
  const int rows_total = SPARSE ? Hq : T * Hq;
  const int n_tiles = (n_keys + kKT - 1) / kKT;

  // ---- this lane's query row (C column = lane % 32) and its Q fragments.  Q.K runs on the
  // FP8 MFMA with the tile's E4M3 key bytes as they are, the bf16 query row scaled by 2^qs
  // and split into two E4M3 terms (bf16x4_split_e4m3: exact for elements at least 2^-9 of
  // the row's largest).  K-step ks, lane half h covers dims 64 ks + 32 h .. + 31, in the
  // same byte order for both operands.
  const int row = row0 + wave * 32 + l32;
  const bool row_ok = row < rows_total;
  const int row_c = row_ok ? row : rows_total - 1;
  const int pos = SPARSE ? 0x7fffffff : (L - T + row_c / Hq);
  i32x8 qhi[kQS], qlo[kQS];
  float sl2;                                          // log2 units per scaled score unit
  {
    const uint16_t* qp = qbase + (size_t)row_c * kDqk + 32 * h;
    u32x4 raw_q[kQS][4];
    uint32_t amax = 0u;
#pragma unroll
    for (int ks = 0; ks < kQS; ++ks)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        raw_q[ks][c] = ld16(qp + 64 * ks + 8 * c);
        amax = bf16x8_absmax_bits(raw_q[ks][c], amax);
      }
    const auto r = __builtin_amdgcn_permlane32_swap(amax, amax, false, false);
    const int qs = split_scale_exp(max(r[0], r[1]));  // the row's largest (both halves)
    const float up = exp2i(qs);
    sl2 = scale_log2 * exp2i(-qs);
#pragma unroll
    for (int ks = 0; ks < kQS; ++ks) {
      uint32_t hw[8], lw[8];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        bf16x4_split_e4m3(raw_q[ks][c].x, raw_q[ks][c].y, up, hw[2 * c], lw[2 * c]);
        bf16x4_split_e4m3(raw_q[ks][c].z, raw_q[ks][c].w, up, hw[2 * c + 1], lw[2 * c + 1]);
      }
      qhi[ks] = as_i32x8(u32x4{hw[0], hw[1], hw[2], hw[3]}, u32x4{hw[4], hw[5], hw[6], hw[7]});
      qlo[ks] = as_i32x8(u32x4{lw[0], lw[1], lw[2], lw[3]}, u32x4{lw[4], lw[5], lw[6], lw[7]});
    }
  }

  // ---- stage validated block ids (decode) or the selections' physical rows (sparse)
  auto sel_row = [&](int idx) -> int {
    if (idx < 0) return -1;
    const int pb = phys_block(bt_row, idx / kBs, n_lblocks, num_blocks);
    return pb >= 0 ? pb * kBs + idx % kBs : -1;
  };
  if constexpr (SPARSE) {
    if constexpr (STAGED) {
      // all of a thread's selections, then all their table entries (at clamped, in-bounds
      // columns), are loaded before any is resolved: two round trips rather than two per
      // selection
      constexpr int kPerT = (kSelLds + NT - 1) / NT;
      int sel[kPerT], ent[kPerT];
#pragma unroll
      for (int u = 0; u < kPerT; ++u) {
        const int j = tid + u * NT;
        sel[u] = j < n_keys ? sel_g[j] : -1;
      }
      if (n_lblocks > 0) {
#pragma unroll
        for (int u = 0; u < kPerT; ++u) ent[u] = bt_row[min(max(sel[u], 0) / kBs, n_lblocks - 1)];
      } else {
#pragma unroll
        for (int u = 0; u < kPerT; ++u) ent[u] = -1;
      }
#pragma unroll
      for (int u = 0; u < kPerT; ++u) {
        const int j = tid + u * NT;
        const int idx = sel[u], pb = ent[u];
        const bool ok = idx >= 0 && idx / kBs < n_lblocks && pb >= 0 && pb < num_blocks;
        const uint32_t r = ok ? (uint32_t)(pb * kBs + idx % kBs) : kNoRow;
        if (j < n_keys) {
          sel_lo[j] = (uint16_t)r;
          sel_hi[j] = (uint8_t)(r >> 16);
        }
      }
    }
  } else {
    for (int j = tid; j < n_bt; j += NT) bt_s[j] = phys_block(bt_row, lb_base + j, n_lblocks, num_blocks);
  }
  __syncthreads();

  // ---- DMA of tile tt into buffer B.  Wave-load j writes LDS bytes 1024 j .. + 1023 of the
  // tile: chunk columns 2 j (lanes 0-31) and 2 j + 1 (lanes 32-63), lane l at slot l % 32 of
  // its column, i.e. key l % 32 ^ 4 (l / 32).  Every load of a lane reads the same key: its
  // row address is computed once per tile, plus the chunk offset 32 j + 16 (l / 32).  (The
  // instruction's immediate offset is not used: on an LDS-DMA it moves the LDS destination
  // too.)
  const uint8_t* zero = kZeroRow;
  asm volatile("" : "+s"(zero));                      // one address, kept in scalar registers
  const int dma_key = l32 ^ (4 * h);
  const int dma_col = 32 * wave + 16 * h;
  // Per tile: prep() resolves the lane's row (tt >= n_tiles: the zero row, so that every
  // step issues the same number of DMA instructions), issues the scale load and writes the
  // valid mask; the kLoadsMax row loads are spread over the next Q.K pass (load()).
  struct Dma {
    const uint8_t* rowp;
    uint32_t dst;
  };
  auto prep = [&](int B, int tt) -> Dma {
    const int kb = tt * kKT;
    const uint32_t dst = lds_u32(&raw[B][0]) + 1024 * wave;
    const uint8_t* rowp;                               // this lane's key row (or zeros)
    const uint8_t* sclp;                               // its scale (used by lanes < 32)
    bool valid;
    if constexpr (SPARSE) {
      const int j = kb + dma_key;
      int q = -1;
      if (j < n_keys) {
        if constexpr (STAGED) {
          const uint32_t r = sel_lo[j] | ((uint32_t)sel_hi[j] << 16);
          q = r == kNoRow ? -1 : (int)r;
        } else {
          q = sel_row(sel_g[j]);
        }
      }
      valid = q >= 0;
      const size_t qb = (size_t)(uint32_t)max(q, 0);
      rowp = valid ? kv + (qb >> 6) * (size_t)blk_bytes + (qb & (kBs - 1)) * kDqk : zero;
      sclp = valid ? ksb + (qb >> 6) * (size_t)sblk_bytes + 4 * (qb & (kBs - 1)) : zero;
    } else {
      const int pos0 = k_begin + kb;
      const int pb = tt < n_tiles ? __builtin_amdgcn_readfirstlane(bt_s[pos0 / kBs - lb_base]) : -1;
      valid = pb >= 0 && kb + dma_key < n_keys;
      const size_t o = (size_t)(pos0 % kBs + dma_key);
      rowp = valid ? kv + (size_t)max(pb, 0) * (size_t)blk_bytes + o * kDqk : zero;
      sclp = valid ? ksb + (size_t)max(pb, 0) * (size_t)sblk_bytes + 4 * o : zero;
    }
    // lanes 0-31 hold keys 0-31 (h = 0: dma_key = lane): the scales and the valid mask
    const uint32_t vmask = (uint32_t)__ballot(h == 0 && valid);
    if (wave == NW - 1) {
      if (h == 0) dma4(sclp, lds_u32(&tsc[B][0]));
      if (lane == 0) tmask[B] = vmask;
    }
    return Dma{rowp + dma_col, dst};
  };
  // Load m of the tile; a wave with fewer loads than kLoadsMax issues a filler load of
  // zeros into `spare` instead (no branch inside the Q.K pass, same count on every wave).
  auto load = [&](const Dma& d, int m) {
    if constexpr (kFiller) {
      const bool real = wave + NW * m < kTileLoads;   // uniform
      dma16((real ? d.rowp : zero + dma_col) + 32 * NW * m, real ? d.dst + 1024 * NW * m : lds_u32(spare));
    } else {
      dma16(d.rowp + 32 * NW * m, d.dst + 1024 * NW * m);
    }
  };
  // DMA instructions this wave issues per tile (the last wave adds the scale load)
  const int my_loads = kLoadsMax + (wave == NW - 1 ? 1 : 0);

  f32x16 acc[kMT];
  // m_run: the row's reference maximum (log2 units), set at its first valid key and fixed;
  // u_max: the largest scaled dot product s * scale_t this lane has seen (its half of the
  // row's keys), checked against m_run + kSlack once, after the last tile
  float m_run = -INFINITY, l_run = 0.f, u_max = -INFINITY;
  bool all_set = false;                               // every row of the wave has its m_run
  // max / sum of a value over lanes l and l ^ 32 (the two halves of a row's keys)
  auto halves = [](float v) {
    return __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  };
  auto halves_max = [&](float v) -> float {
    const auto r = halves(v);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  };
  auto halves_sum = [&](float v) -> float {
    const auto r = halves(v);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  };

  // per-lane LDS offsets (bytes, relative to a tile)
  // V^T fragment of output tile mt, key step kk: within each 16-lane group g = lane / 16,
  // source lane s = 2 k + hh reads key 16 kk + 4 (g / 2) + k + 4 (k / 4) at bytes
  // 32 mt + 16 (g % 2) + 8 hh (chunk 2 mt + g % 2); the lane then holds dim 32 mt + lane % 32
  // of keys 16 kk + 4 h + {0..3, 8..11} -- the keys of its P fragment.
  const int vg = lane >> 4, vs = lane & 15, vk = vs >> 1, vhh = vs & 1;
  const int v_key0 = 4 * (vg >> 1) + vk + 4 * (vk >> 2);
  const int v_base = (vg & 1) * kColB + 16 * (v_key0 ^ (4 * (vg & 1))) + 8 * vhh;   // + 256 kk + 1024 mt
  lds_u8* const lds = (lds_u8*)&raw[0][0];

  // S^T = K Q^T over the 9 k-steps of tile buffer B, two FP8 MFMAs each (Q's hi and lo terms),
  // the key bytes fed as read; fragment reads kPre / 4 k-steps ahead, and the row loads of
  // the next tile spread over the 18 MFMAs.  K-step ks of lane half h reads chunks
  // 4 ks + 2 h (even: key l32 in place) and 4 ks + 2 h + 1 (odd: key l32 ^ 4).
  auto qk = [&](int B, const Dma& d) -> f32x16 {
    const int tk = B * kTileB + 2 * h * kColB;
    const int k_even = 16 * l32, k_odd = kColB + 16 * (l32 ^ 4);
    f32x16 s0;
#pragma unroll
    for (int i = 0; i < 16; ++i) s0[i] = 0.f;
    constexpr int kPreK = kPre / 4;                    // k-steps of reads in flight
    u32x4 kr[kPreK][2];
#pragma unroll
    for (int j = 0; j < kPreK; ++j) {
      kr[j][0] = lds_read_b128(lds, tk + 4 * j * kColB + k_even);
      kr[j][1] = lds_read_b128(lds, tk + 4 * j * kColB + k_odd);
    }
    constexpr int kMf = 2 * kQS;                       // MFMAs per tile
    constexpr int kEvery = kMf / kLoadsMax;
#pragma unroll
    for (int ks = 0; ks < kQS; ++ks) {
      const i32x8 ka = as_i32x8(kr[ks % kPreK][0], kr[ks % kPreK][1]);
      const int n = ks + kPreK;
      if (n < kQS) {
        kr[ks % kPreK][0] = lds_read_b128(lds, tk + 4 * n * kColB + k_even);
        kr[ks % kPreK][1] = lds_read_b128(lds, tk + 4 * n * kColB + k_odd);
      }
#pragma unroll
      for (int term = 0; term < 2; ++term) {
        s0 = mfma32x32x64_fp8(ka, term ? qlo[ks] : qhi[ks], s0);
        const int i = 2 * ks + term;
        if (i % kEvery == kEvery / 2 && i / kEvery < kLoadsMax) load(d, i / kEvery);
      }
    }
    return s0;
  };
  // O^T += V^T P^T over tile buffer B (fragment reads kPre ahead)
  auto pv = [&](int B, const u32x4 (&pb)[2]) {
    const int tv = B * kTileB + v_base;
    u32x2 vr[kPre];
#pragma unroll
    for (int j = 0; j < kPre; ++j) vr[j] = lds_read_tr8(lds, tv + 256 * (j / kMT) + 1024 * (j % kMT));
#pragma unroll
    for (int i = 0; i < 2 * kMT; ++i) {
      const int kk = i / kMT, mt = i % kMT;
      const u32x2 vc = vr[i % kPre];
      const int n = i + kPre;
      if (n < 2 * kMT) vr[i % kPre] = lds_read_tr8(lds, tv + 256 * (n / kMT) + 1024 * (n % kMT));
      acc[mt] = mfma32x32x16_f16(fp8x8_to_f16x8(vc), pb[kk], acc[mt]);
    }
  };
  // scale, mask and softmax of tile t (buffer B); lane holds row `row`, keys 8 (i / 4) +
  // 4 h + i % 4; P as fp16 B operands, k-step kk holding keys 16 kk + 8 (j / 4) + 4 h + j % 4
  //
  // Once every row of the wave has its reference (all_set, usually from the first tile on)
  // the softmax is elementwise: no reduction across lanes, no guard for a row without one,
  // and no clamp -- a row whose p would pass 2^kSlack is caught by the v_max check at the
  // end, and its work unit is recomputed exactly, so what it accumulated is never used.
  // Tiles whose keys are all visible (the common case) skip the mask.
  // In log2 units a score is v = u * sl2 with u = s * scale_t (s in the query's scaled units,
  // sl2 = scale_log2 * 2^-qs), and p = 2^(v - m_run) is evaluated as exp2(fma(u, sl2, -m_run)).
  auto softmax = [&](int B, int t, const f32x16& s0, u32x4 (&pb)[2]) {
    uint32_t okm = tmask[B];
    if constexpr (!SPARSE) {
      const int lim = pos - (k_begin + t * kKT) + 1;  // causal: keys k < lim are visible
      okm &= lim >= 32 ? ~0u : (lim <= 0 ? 0u : ((1u << lim) - 1u));
    }
    const bool full = __ballot(okm != ~0u) == 0;     // every row sees all 32 keys
    okm >>= 4 * h;
    // this lane's keys 8 q4 + 4 h + i: scales, then u (masked keys -inf)
    f32x4 sc[4];
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) sc[q4] = *reinterpret_cast<const f32x4*>(&tsc[B][8 * q4 + 4 * h]);
    float u[16];
    if (full) {
#pragma unroll
      for (int i = 0; i < 16; ++i) u[i] = s0[i] * sc[i / 4][i % 4];
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        u[i] = ((okm >> (8 * (i / 4) + i % 4)) & 1u) ? s0[i] * sc[i / 4][i % 4] : -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, u[i]);
    u_max = fmaxf(u_max, mx);
    float m_sub = m_run;
    if (!all_set) {
      // some row still lacks a reference: take it from this tile's row maximum (a row with
      // no visible key so far keeps -inf, and its p are 0)
      const float row_mx = halves_max(mx);
      if (m_run == -INFINITY) m_run = row_mx * sl2;
      m_sub = m_run == -INFINITY ? 0.f : m_run;
      all_set = __ballot(m_run == -INFINITY) == 0;
    }
    float rs = 0.f;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      float pvv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        // masked keys: p = exp2(-inf) = 0; invalid keys also have a zero scale and zero V
        const int i = 8 * kk + j;
        const float p = fast_exp2(__builtin_fmaf(u[i], sl2, -m_sub));
        rs += p;
        pvv[j] = p * sc[i / 4][i % 4];
      }
      pb[kk] = u32x4{pack_f16x2(pvv[0], pvv[1]), pack_f16x2(pvv[2], pvv[3]), pack_f16x2(pvv[4], pvv[5]),
                     pack_f16x2(pvv[6], pvv[7])};
    }
    l_run += rs;
  };

#pragma unroll
  for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[mt][i] = 0.f;
  // ---- pipeline: buffer t % NBUF holds tile t; tile t + NBUF - 1 is issued at step t into
  // the buffer tile t - 1 used, after the barrier that ends every wave's use of it.  Every
  // step issues my_loads DMA instructions (zero rows past the last tile), so before step t
  // exactly (NBUF - 2) * my_loads of them follow tile t's.
#pragma unroll
  for (int i = 0; i < NBUF - 1; ++i) {
    const Dma d = prep(i, i);
#pragma unroll
    for (int m = 0; m < kLoadsMax; ++m) load(d, m);
  }
  for (int t = 0; t < n_tiles; ++t) {
    // this wave's DMA of tile t has landed
    wait_vm_upto<(NBUF - 2) * (kLoadsMax + 1)>((NBUF - 2) * my_loads);
    barrier_lds();
    const int B = t % NBUF;
    const Dma d = prep((t + NBUF - 1) % NBUF, t + NBUF - 1);
    u32x4 pb[2];
    const f32x16 s0 = qk(B, d);
    softmax(B, t, s0, pb);
    pv(B, pb);
  }
  wait_vm<0>();                                       // no DMA outlives the workgroup
  {
    const float row_umax = halves_max(u_max);
    const bool ovf = m_run != -INFINITY && __builtin_fmaf(row_umax, sl2, -m_run) > kSlack;
    const bool w_ovf = __ballot(ovf) != 0;
    if (lane == 0) ovf_s[wave] = w_ovf ? 1 : 0;
  }
  barrier_lds();
  bool overflow = false;
#pragma unroll
  for (int w = 0; w < NW; ++w) overflow |= ovf_s[w] != 0;

  // ---- finish: full row sum over the two lane halves, write the 32 rows x 512 dims.  The
  // lane's row and half are derived again here (from the lane id, counted with mbcnt) rather
  // than kept in registers through the tile loop.
  const float l_tot = halves_sum(l_run);
  const int lane_e = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  const int row_e = row0 + wave * 32 + (lane_e & 31), h_e = lane_e >> 5;
  if (row_e >= rows_total) return;
  if (overflow) {
    // mark the unit for the exact recomputation: a NaN in every row's LSE (decode) or in
    // the first output element of every row (sparse)
    if (h_e == 0) {
      if constexpr (SPARSE) sa.out[((size_t)unit * Hq + row_e) * kDv] = 0x7fc1;
      else da.part_lse[((size_t)unit * da.max_splits + unit_split) * rows_total + row_e] = __builtin_nanf("");
    }
    return;
  }
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const float lse2 = l_tot > 0.f ? m_run + __log2f(l_tot) : -INFINITY;
  // acc[mt][4 q + i] = O[row][32 mt + 8 q + 4 h + i]
  if constexpr (SPARSE) {
    uint16_t* op = sa.out + ((size_t)unit * Hq + row_e) * kDv + 4 * h_e;
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        u32x2 w;
        w.x = pack_bf16x2(acc[mt][4 * q] * inv, acc[mt][4 * q + 1] * inv);
        w.y = pack_bf16x2(acc[mt][4 * q + 2] * inv, acc[mt][4 * q + 3] * inv);
        *reinterpret_cast<u32x2*>(op + 32 * mt + 8 * q) = w;
      }
    if (sa.lse != nullptr && h_e == 0) sa.lse[(size_t)unit * Hq + row_e] = lse2 == -INFINITY ? -INFINITY : lse2 * kLn2;
  } else {
    const size_t pbase = ((size_t)unit * da.max_splits + unit_split) * rows_total + row_e;
    float* op = da.part_o + pbase * kDv + 4 * h_e;
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<f32x4*>(op + 32 * mt + 8 * q) =
            f32x4{acc[mt][4 * q], acc[mt][4 * q + 1], acc[mt][4 * q + 2], acc[mt][4 * q + 3]} * inv;
    if (h_e == 0) da.part_lse[pbase] = lse2;
  }
}

#ifndef PA_MLA2_DECODE_NBUF
#define PA_MLA2_DECODE_NBUF 4
#endif
#ifndef PA_MLA2_SPARSE_NBUF
#define PA_MLA2_SPARSE_NBUF 4
#endif
constexpr int kDecWaves = 4, kSpWaves = 2;
constexpr int kDecBuf = PA_MLA2_DECODE_NBUF, kSpBuf = PA_MLA2_SPARSE_NBUF;

}  // namespace

hipError_t launch_mla_decode(const MlaDecodeArgs& a, hipStream_t stream) {
  const int rows = a.q_per_seq * a.num_q_heads;
  const unsigned grid = (unsigned)a.num_seqs * a.max_splits * ((rows + 32 * kDecWaves - 1) / (32 * kDecWaves));
  if (grid == 0) return hipSuccess;
  SparseMlaArgs none{};
  hipLaunchKernelGGL((mla_kernel<false, kDecWaves, kDecBuf, false>), dim3(grid), dim3(64 * kDecWaves), 0, stream, a,
                     none);
  const hipError_t e = hipGetLastError();
  return e != hipSuccess ? e : launch_mla_decode_exact(a, stream);
}

hipError_t launch_sparse_mla(const SparseMlaArgs& a, hipStream_t stream) {
  const unsigned grid = (unsigned)a.n_q * ((a.num_q_heads + 32 * kSpWaves - 1) / (32 * kSpWaves));
  if (grid == 0) return hipSuccess;
  MlaDecodeArgs none{};
  if (a.k <= kSelLds && (int64_t)a.num_blocks * kBs < (int64_t)kNoRow)
    hipLaunchKernelGGL((mla_kernel<true, kSpWaves, kSpBuf, true>), dim3(grid), dim3(64 * kSpWaves), 0, stream, none, a);
  else
    hipLaunchKernelGGL((mla_kernel<true, kSpWaves, kSpBuf, false>), dim3(grid), dim3(64 * kSpWaves), 0, stream, none, a);
  const hipError_t e = hipGetLastError();
  return e != hipSuccess ? e : launch_sparse_mla_exact(a, stream);
}

}  // namespace pa
