// MLA attention over the FP8 latent cache, the exact two-stage form: paged decode (with MTP
// query tokens) and sparse MLA over indexer-selected tokens.  It recomputes the work units
// that the main MLA kernel (mla.hip) marked -- those where a row's running maximum moved too
// far for its fixed reference -- with the rescaling online softmax; every other unit
// returns at once.
//
// Sources: vLLM AgentX article (news.ainew.jp), "Kimi K3" (MLA keeps one latent head;
// partial outputs merged by log-sum-exp) and "DeepSeek V4" (sparse MLA gathers the top-k
// KV entries, then attends); GLM-5.3 report (aisoku.org), "What's new" (the latent KV is
// shared by all 64 heads), its table (FP8 KV, MTP3) and "How to try" (prompts inside the
// top-k use the same sparse MQA kernel).
//
// The latent is shared by every query head, so attention is MQA with d_qk = 576 (512
// latent + 64 rope) and d_v = 512 (the latent itself).  A workgroup holds NP wave pairs;
// pair p owns 32 query rows and every pair reads the same keys (decode: 4 pairs = 128
// rows, e.g. two MTP tokens x 64 heads; sparse: two groups of four waves = the 64 heads of
// one query, each wave a quarter of the dimensions).
// Keys go in 32-key tiles through a three-stage pipeline:
//   1. LDS-DMA (global_load_lds, 16 bytes a lane) gathers tile t+2's FP8 rows through the
//      block table into a raw LDS buffer -- no registers held while the loads fly.  Decode
//      stages its range's block ids in LDS once; sparse resolves every selected position
//      to its physical row (block * 64 + offset) once and stages the rows, so the DMA of
//      a tile waits for no table lookup.
//   2. All threads upcast tile t+1's raw bytes once, exactly, to fp16 into a row-major
//      LDS tile (16-byte chunks XOR-swizzled by row/4: conflict-free for both read
//      patterns below); keys that are invalid (past the range, unselected, bad block id)
//      become zeros, so stale bytes can never inject NaN.
//   3. Tile t is computed from the fp16 tile with v_mfma_f32_32x32x16_f16.  The two
//      waves of a pair split the work instead of duplicating it: for S^T = K Q^T each
//      contracts one half of the 576 dims (Q half in 72 VGPRs) and the partial 32x32
//      tiles are exchanged through LDS and added in a fixed order, so both waves hold the
//      same S; for O^T += V^T P^T each wave owns 256 of the 512 output dims (128
//      accumulator registers), reading V^T fragments with ds_read_b64_tr_b16.
// The per-token fp32 scale multiplies the scores (s = scale_t q.k) and the probabilities
// used for P.V (p * scale_t), never the staged fp16 values; queries are converted once
// from bf16 to fp16 (exact for |q| in [2^-14, 65504]).  Online softmax per row; the
// accumulator is rescaled only when a row's running maximum grows.
#include <type_traits>


#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

#ifndef PA_MLA_SPARSE_XCD
#define PA_MLA_SPARSE_XCD 1
#endif
constexpr int kDqk = 576, kDv = 512, kBs = 64;
constexpr int kKT = 32;                   // keys per tile
constexpr int kKS = 608;                  // fp16 per LDS row: 1,216 B, 304 dwords = 48 mod 64
constexpr int kChunks = kKT * (kDqk / 16);   // 16-byte FP8 chunks per tile (1,152)
constexpr int kWaveLoads = kChunks / 64;     // 1 KB DMA wave-loads per tile (18)
constexpr int kSelLds = 2048;             // selected positions staged in LDS (sparse)
static_assert(kChunks % 64 == 0, "tile is a whole number of wave-loads");
static_assert(kKS >= kDqk + 16, "row 0's padding takes the discarded chunk slots");

template <int N>
using Int = std::integral_constant<int, N>;

// NW waves per workgroup; SPLIT waves share each group of 32 query rows (1: a wave holds
// all 576 Q dims and all 512 output dims; 2 or 4: the waves split both, exchanging
// partial S through LDS).  STAGED (sparse only): the physical rows of the selections
// (k <= 2048) are resolved once and kept in LDS; otherwise every tile resolves its keys
// from global memory (a separate instantiation, so no lookup ever becomes a flat access).  LATE_CONV: the upcast of tile t+1 runs interleaved with the P.V of tile
// t (pays off with one wave a SIMD and registers to spare) instead of at the start of
// step t.
template <bool SPARSE, int NW, int SPLIT, bool STAGED, bool LATE_CONV, bool REDO>
__global__ __launch_bounds__(NW * 64, 1) void mla_kernel(MlaDecodeArgs da, SparseMlaArgs sa) {
  constexpr int NT = NW * 64;
  constexpr int RW = 32 * NW / SPLIT;       // query rows per workgroup
  constexpr int kQW = 36 / SPLIT;           // QK k-steps of 16 dims per wave
  constexpr int kMW = 16 / SPLIT;           // O^T tiles of 32 dims per wave
  static_assert(SPLIT == 1 || SPLIT == 2 || SPLIT == 4, "split");
  // The raw DMA targets are LDS objects of their own: the compiler then knows that reads
  // of the fp16 tiles (and of the other raw buffer) never alias a buffer the DMA is
  // filling, and inserts no wait for them.
  __shared__ __attribute__((aligned(16))) uint16_t fb[2][kKT * kKS];
  __shared__ __attribute__((aligned(16))) uint8_t r0[kKT * kDqk];
  __shared__ __attribute__((aligned(16))) uint8_t r1[kKT * kDqk];
  __shared__ __attribute__((aligned(16))) float rs0[kKT];
  __shared__ __attribute__((aligned(16))) float rs1[kKT];
  __shared__ __attribute__((aligned(16))) int32_t rk0[kKT];
  __shared__ __attribute__((aligned(16))) int32_t rk1[kKT];
  __shared__ __attribute__((aligned(16))) int32_t fk[2][kKT];    // position, -1 if invalid
  __shared__ __attribute__((aligned(16))) float fks[2][kKT];     // scale * softmax scale * log2 e
  __shared__ __attribute__((aligned(16))) float fvs[2][kKT];     // scale
  __shared__ int32_t fall[2];                                    // 1: every key of the tile valid
  __shared__ __attribute__((aligned(16))) f32x4 xs[SPLIT > 1 ? NW * 4 * 64 : 1];  // partial S
  // decode stages its range's block ids; sparse stages, per selection, the physical row
  // (block * 64 + offset, or -1) resolved through the block table once per workgroup
  __shared__ int32_t bt_s[SPARSE ? 1 : kDecodeSplitMla / kBs + 1];
  __shared__ int32_t sel_s[SPARSE && STAGED ? kSelLds : 1];
  // Decode (two waves a SIMD) keeps its first Q fragment in LDS, one 16-byte read per tile,
  // instead of a register: the register file is the limit there, and a spilled fragment
  // would be reloaded from scratch memory inside the pipeline.
  constexpr int kQL = SPARSE ? 0 : 1;
  __shared__ __attribute__((aligned(16))) u32x4 qls[kQL > 0 ? kQL * NT : 1];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: keep it scalar
  const int l32 = lane & 31, h = lane >> 5;
  const int grp32 = wave / SPLIT;                    // which 32 rows
  const int half = wave % SPLIT;                     // which share of the dims

  // ---- work unit
  const uint16_t* qbase;
  const int32_t* bt_row;
  const int32_t* sel_g = nullptr;
  const uint8_t* kv;
  const uint8_t* ksb;                               // latent scales (see MlaDecodeArgs)
  int64_t blk_bytes, sblk_bytes;
  int Hq, n_keys, k_begin = 0, n_lblocks, L = 0, T = 1, row0, unit = 0, unit_split = 0;
  int lb_base = 0, n_bt, num_blocks;
  float scale_log2;
  if constexpr (SPARSE) {
    Hq = sa.num_q_heads;
    const int rblocks = (Hq + RW - 1) / RW;
    // consecutive query tokens select overlapping keys: keep them on one XCD (shared L2)
    const int bid = PA_MLA_SPARSE_XCD ? xcd_swizzle(blockIdx.x, gridDim.x) : (int)blockIdx.x;
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
    n_bt = 0;
    scale_log2 = sa.scale_log2;
  } else {
    Hq = da.num_q_heads;
    T = da.q_per_seq;
    const int rows = T * Hq;
    const int rblocks = (rows + RW - 1) / RW;
    const int n_units = da.num_seqs * da.max_splits * rblocks;
    // (sequence, split) units go to the XCDs round robin, with each sequence's split order
    // rotated by its index: every XCD gets about 1/8 of every sequence's keys, whatever the
    // mix of context lengths (the row blocks of a unit share its XCD's L2)
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
    n_bt = (k_begin + n_keys + kBs - 1) / kBs - lb_base;   // <= kDecodeSplitMla / kBs
    scale_log2 = da.scale_log2;
  }
  const int rows_total = SPARSE ? Hq : T * Hq;
  if constexpr (REDO) {
    // recompute only the units the fixed-reference kernel marked (a NaN in the first
    // row's LSE, or in its first output element for sparse)
    if constexpr (SPARSE) {
      const uint16_t b = sa.out[((size_t)unit * Hq + row0) * kDv];
      if ((b & 0x7f80u) != 0x7f80u || (b & 0x7fu) == 0) return;
    } else {
      const float m = da.part_lse[((size_t)unit * da.max_splits + unit_split) * rows_total + row0];
      if (!(m != m)) return;
    }
  }

  // ---- this lane's query row (C column = lane % 32) and its fp16 Q fragments
  const int row = row0 + grp32 * 32 + l32;
  const bool row_ok = row < rows_total;
  const int row_c = row_ok ? row : rows_total - 1;
  const int pos = SPARSE ? 0x7fffffff : (L - T + row_c / Hq);
  u32x4 qb[kQW];
  {
    const uint16_t* qp = qbase + (size_t)row_c * kDqk + 16 * kQW * half + 8 * h;
#pragma unroll
    for (int ks = 0; ks < kQW; ++ks) {
      const u32x4 v = ld16(qp + 16 * ks);
      const u32x4 f = u32x4{bf16x2_to_f16x2(v.x), bf16x2_to_f16x2(v.y), bf16x2_to_f16x2(v.z), bf16x2_to_f16x2(v.w)};
      if (ks < kQL)
        qls[ks * NT + tid] = f;
      else
        qb[ks] = f;
    }
  }

  // ---- stage validated block ids (decode) or the selections' physical rows (sparse)
  // j-th selection -> physical row of the pool (block * 64 + offset), -1 if unselected or
  // its block id is out of range (rows fit in 32 bits: the library checks num_blocks)
  auto sel_row = [&](int idx) -> int {
    if (idx < 0) return -1;
    const int pb = phys_block(bt_row, idx / kBs, n_lblocks, num_blocks);
    return pb >= 0 ? pb * kBs + idx % kBs : -1;
  };
  for (int j = tid; j < n_bt; j += NT) bt_s[j] = phys_block(bt_row, lb_base + j, n_lblocks, num_blocks);
  if constexpr (SPARSE && STAGED) {
    for (int j = tid; j < n_keys; j += NT) sel_s[j] = sel_row(sel_g[j]);
  }
  __syncthreads();
  // sparse: j-th key of the unit -> physical row, or -1
  auto key_row = [&](int j) -> int {
    if (j >= n_keys) return -1;
    if constexpr (STAGED) return sel_s[j];
    else return sel_row(sel_g[j]);
  };

  // ---- stage 1: DMA tile tt into raw buffer P.  Raw chunk c (16 bytes: key c / 36,
  // dims 16 (c % 36) ..) lands at R + 16 c; wave-load j covers chunks 64 j .. 64 j + 63.
  constexpr int kLoadsPerWave = (kWaveLoads + NW - 1) / NW;
  auto issue = [&](auto P, int tt) {
    uint8_t* R = P ? r1 : r0;
    float* RS = P ? rs1 : rs0;
    int32_t* RK = P ? rk1 : rk0;
    const int kb = tt * kKT;
    int ln = lane;
    asm volatile("" : "+v"(ln));   // recompute the lane's indices here, keep no VGPRs for them
    if constexpr (!SPARSE) {
      // a 32-key tile of a contiguous range never straddles a 64-token block: its FP8
      // rows are one contiguous 18,432-byte span of one block
      const int pos0 = k_begin + kb;
      const int pb = bt_s[pos0 / kBs - lb_base];
      const uint8_t* span = pb >= 0 ? kv + (size_t)pb * blk_bytes + (pos0 % kBs) * kDqk : kv;
#pragma unroll
      for (int m = 0; m < kLoadsPerWave; ++m) {
        const int j = wave + NW * m;
        if (j < kWaveLoads) dma16(pb >= 0 ? span + 16 * (64 * j + ln) : kv, lds_u32(R) + 1024 * j);
      }
      if (wave == NW - 1 && ln < kKT) {
        dma4(pb >= 0 ? reinterpret_cast<const float*>(ksb + (size_t)pb * sblk_bytes) + pos0 % kBs + ln
                     : reinterpret_cast<const float*>(ksb), lds_u32(RS));
        RK[ln] = (pb >= 0 && kb + ln < n_keys) ? pos0 + ln : -1;
      }
    } else {
      // per-key rows, all LDS reads issued before the DMAs; a valid key's RK entry is its
      // physical row (>= 0: the only property the sparse path reads)
      int prow[kLoadsPerWave];
#pragma unroll
      for (int m = 0; m < kLoadsPerWave; ++m) {
        const int key = (64 * (wave + NW * m) + ln) / (kDqk / 16);
        prow[m] = key_row(kb + key);
      }
#pragma unroll
      for (int m = 0; m < kLoadsPerWave; ++m) {
        const int j = wave + NW * m;
        const int dc = (64 * j + ln) % (kDqk / 16);
        const int pr = prow[m];
        if (j < kWaveLoads)
          dma16(pr >= 0 ? kv + (size_t)(pr >> 6) * blk_bytes + (pr & (kBs - 1)) * kDqk + 16 * dc : kv,
                lds_u32(R) + 1024 * j);
      }
      if (wave == NW - 1 && ln < kKT) {
        const int pr = key_row(kb + ln);
        dma4(pr >= 0 ? reinterpret_cast<const float*>(ksb + (size_t)(pr >> 6) * sblk_bytes) + (pr & (kBs - 1))
                     : reinterpret_cast<const float*>(ksb), lds_u32(RS));
        RK[ln] = pr;
      }
    }
  };
  // ---- stage 2: raw buffer P -> fp16 tile P, unrolled with all LDS reads first.  With the
  // late upcast it is also branch-free, so that it shares a basic block with -- and
  // interleaves with -- the P.V MFMAs of the previous tile: chunk slots past the tile
  // then write into row 0's padding (fp16 576 .. 591), which nothing reads.
  constexpr int CPT = (kChunks + NT - 1) / NT;
  auto convert_chunks = [&](auto P) {
    const uint8_t* R = P ? r1 : r0;
    const int32_t* RK = P ? rk1 : rk0;
    uint16_t* F = fb[P];
    int th = tid;
    asm volatile("" : "+v"(th));
    u32x4 raw[CPT];
    bool ok[CPT];
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = th + NT * i;
      const bool in = i < CPT - 1 || c < kChunks;
      const int cc = in ? c : 0;
      ok[i] = in && RK[cc / (kDqk / 16)] >= 0;
      raw[i] = *reinterpret_cast<const u32x4*>(R + 16 * cc);
    }
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = th + NT * i;
      const bool in = i < CPT - 1 || c < kChunks;
      const int key = c / (kDqk / 16), dc = c % (kDqk / 16);
      const int v = (key >> 2) & 3;
      const u32x2 a0 = fp8x4_to_f16x4(raw[i].x), a1 = fp8x4_to_f16x4(raw[i].y);
      const u32x2 a2 = fp8x4_to_f16x4(raw[i].z), a3 = fp8x4_to_f16x4(raw[i].w);
      const u32x4 lo = ok[i] ? u32x4{a0.x, a0.y, a1.x, a1.y} : u32x4{0, 0, 0, 0};
      const u32x4 hi = ok[i] ? u32x4{a2.x, a2.y, a3.x, a3.y} : u32x4{0, 0, 0, 0};
      if constexpr (LATE_CONV) {   // branch-free: the discarded slots go to the padding
        const int o_lo = in ? key * kKS + 8 * ((2 * dc) ^ v) : kDqk;
        const int o_hi = in ? key * kKS + 8 * ((2 * dc + 1) ^ v) : kDqk + 8;
        st16(F + o_lo, lo);
        st16(F + o_hi, hi);
      } else if (in) {
        st16(F + key * kKS + 8 * ((2 * dc) ^ v), lo);
        st16(F + key * kKS + 8 * ((2 * dc + 1) ^ v), hi);
      }
    }
  };
  // key metadata of the tile in raw buffer P -> fp16 tile P's metadata (wave 0)
  auto convert_meta = [&](auto P) {
    const float* RS = P ? rs1 : rs0;
    const int32_t* RK = P ? rk1 : rk0;
    if (wave == 0) {
      int ln = lane;
      asm volatile("" : "+v"(ln));   // recompute the addresses here, keep no VGPRs for them
      const int id = ln < kKT ? RK[ln] : 0;
      const float sc = ln < kKT ? RS[ln] : 0.f;
      if (ln < kKT) {
        fk[P][ln] = id;
        fks[P][ln] = id >= 0 ? sc * scale_log2 : 0.f;
        fvs[P][ln] = id >= 0 ? sc : 0.f;
      }
      const bool all_valid = __ballot(id < 0) == 0;
      if (ln == 0) fall[P] = all_valid ? 1 : 0;
    }
  };
  auto convert = [&](auto P) {
    convert_chunks(P);
    convert_meta(P);
  };

  // ---- per-lane LDS offsets (fp16 units) into an fp16 tile, swizzle folded in.  They are
  // recomputed from an opaque copy of the lane id where each phase starts, so that none
  // of them holds a register through the other phases (the register file is the limit).
  auto fresh_lane = []() -> int {
    int ln = (int)__lane_id();
    asm volatile("" : "+v"(ln));
    return ln;
  };
  // K fragment of k-step ks (0..35): key row l32, logical chunk 2ks + h stored at chunk
  // (2ks + h) ^ v, v = (l32 / 4) & 3; ks parity decides the sign of the v/2 term.  The
  // pair (even-step base, odd-step base) is swapped when this wave's first step is odd.
  auto k_bases = [&](int& k_even, int& k_odd) {
    const int ln = fresh_lane();
    const int r = ln & 31, hh = ln >> 5, vk = (r >> 2) & 3;
    const int base = r * kKS + 8 * (hh ^ (vk & 1));
    k_even = base + 16 * (vk >> 1);
    k_odd = base - 16 * (vk >> 1);
    if ((kQW * half) & 1) {
      const int t = k_even; k_even = k_odd; k_odd = t;
    }
  };
  // V^T fragments of k-step kk and output tile mt: rows 16kk + 4h + n/4 (first read) and
  // 8 rows further (second), logical chunk 4mt + 2(g%2) + (n%4)/2, fp16 offset 4(n&1).
  auto v_bases = [&](int& v_lo, int& v_hi) {
    const int ln = fresh_lane();
    const int hh = ln >> 5, gg = ln >> 4, n = ln & 15;
    const int vrow = 4 * hh + (n >> 2);
    const int vsub = 2 * (gg & 1) + ((n & 3) >> 1);
    v_lo = vrow * kKS + 8 * (vsub ^ hh) + 4 * (n & 1);
    v_hi = (vrow + 8) * kKS + 8 * (vsub ^ ((hh + 2) & 3)) + 4 * (n & 1);
  };
  // this wave's S share slot, and the first share of its pair
  auto x_own = [&]() -> f32x4* { return xs + (SPLIT > 1 ? wave * 256 + fresh_lane() : 0); };
  auto x_pair = [&]() -> const f32x4* { return xs + (SPLIT > 1 ? (wave - half) * 256 + fresh_lane() : 0); };
  auto x_partner = [&]() -> const f32x4* { return xs + (SPLIT == 2 ? (wave ^ 1) * 256 + fresh_lane() : 0); };

  f32x16 acc[kMW];
#pragma unroll
  for (int mt = 0; mt < kMW; ++mt)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[mt][i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  // Max / sum of a value over lanes l and l ^ 32, without an LDS round trip and without
  // the lane id: after the swap one copy holds the low half's values in both halves and
  // the other the high half's, so every lane combines the same two operands in the same
  // order.
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

  // ---- stage 3a: S^T[32 keys x 32 rows] over this wave's share of the 576 dims
  auto qk = [&](auto P) -> f32x16 {
    const uint16_t* F = fb[P];
    int k_even, k_odd;
    k_bases(k_even, k_odd);
    f32x16 s;
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = 0.f;
    if constexpr (SPARSE) {
      // registers to spare here: every K fragment is read before the MFMAs, so the reads
      // are in flight together instead of two at a time
      u32x4 kf[kQW];
#pragma unroll
      for (int k = 0; k < kQW; ++k)
        kf[k] = *reinterpret_cast<const u32x4*>(F + ((k & 1) ? k_odd : k_even) + 16 * (kQW * half + k));
#pragma unroll
      for (int k = 0; k < kQW; ++k) s = mfma32x32x16_f16(kf[k], k < kQL ? qls[k * NT + tid] : qb[k], s);
      __builtin_amdgcn_sched_group_barrier(0x100, kQW, 0);   // the K reads first
      __builtin_amdgcn_sched_group_barrier(0x008, kQW, 0);   // then the MFMAs
    } else {
#pragma unroll
      for (int k = 0; k < kQW; ++k) {
        const int ks = kQW * half + k;             // bases swapped above when kQW * half is odd
        const uint16_t* kp = F + ((k & 1) ? k_odd : k_even) + 16 * ks;
        s = mfma32x32x16_f16(*reinterpret_cast<const u32x4*>(kp), k < kQL ? qls[k * NT + tid] : qb[k], s);
      }
    }
    return s;
  };
  // ---- stage 3b: full S, online softmax, O^T += V^T P^T for this wave's output dims
  auto softmax_pv = [&](auto P, f32x16 s_in, int t, bool conv_next) {
    const uint16_t* F = fb[P];
    // scalars, not a 16-register tuple: per-element updates then need no tuple copies
    float s[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = s_in[i];
    if constexpr (SPLIT == 2) {
      // the full S = own share + partner's share; float addition is commutative, so both
      // waves of the pair get bit-identical sums
      const f32x4* xq = x_partner();
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const f32x4 b = xq[64 * i4];
#pragma unroll
        for (int i = 0; i < 4; ++i) s[4 * i4 + i] += b[i];
      }
    } else if constexpr (SPLIT == 4) {
      // rebuild the full S from all published shares in one fixed order -- the same
      // operations in every wave of the group
      const f32x4* xp = x_pair();
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const f32x4 a = xp[64 * i4], b = xp[256 + 64 * i4];
        const f32x4 sum = (a + b) + (xp[512 + 64 * i4] + xp[768 + 64 * i4]);
#pragma unroll
        for (int i = 0; i < 4; ++i) s[4 * i4 + i] = sum[i];
      }
    }
    // scale (and mask where needed); lane holds row `row`, keys 8(i/4) + 4h + i%4.  A tile
    // needs no mask when every key is valid and (decode) even its last key is at or below
    // the earliest query position.
    const bool interior = fall[P] != 0 && (SPARSE || k_begin + t * kKT + kKT - 1 <= L - T);
    float mx = -INFINITY;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int kb4 = 8 * q4 + 4 * h;
      const f32x4 ksc = *reinterpret_cast<const f32x4*>(&fks[P][kb4]);
      if (interior) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          s[4 * q4 + i] *= ksc[i];
          mx = fmaxf(mx, s[4 * q4 + i]);
        }
      } else {
        const int4 id = *reinterpret_cast<const int4*>(&fk[P][kb4]);
        const int idv[4] = {id.x, id.y, id.z, id.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float v = (idv[i] >= 0 && idv[i] <= pos) ? s[4 * q4 + i] * ksc[i] : -INFINITY;
          s[4 * q4 + i] = v;
          mx = fmaxf(mx, v);
        }
      }
    }
    mx = halves_max(mx);
    // The reference maximum moves only when a row's maximum grows by more than 2^8
    // (log2 units): probabilities stay <= 256, exact enough in fp16, and the accumulator
    // is rescaled almost never.  Softmax does not depend on the reference.
    if (__ballot(mx > m_run + 8.f) != 0) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = m_run == -INFINITY ? 0.f : fast_exp2(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int mt = 0; mt < kMW; ++mt) acc[mt] *= alpha;
      m_run = m_new;
    }
    // probabilities -> fp16 B operands; k-step kk holds keys 16kk + 8(j/4) + 4h + j%4
    float rs = 0.f;
    u32x4 pb[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      float pv[8];
#pragma unroll
      for (int q2 = 0; q2 < 2; ++q2) {
        const f32x4 vsc = *reinterpret_cast<const f32x4*>(&fvs[P][16 * kk + 8 * q2 + 4 * h]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = m_run == -INFINITY ? 0.f : fast_exp2(s[8 * kk + 4 * q2 + i] - m_run);
          rs += p;
          pv[4 * q2 + i] = p * vsc[i];
        }
      }
      pb[kk] = u32x4{pack_f16x2(pv[0], pv[1]), pack_f16x2(pv[2], pv[3]),
                     pack_f16x2(pv[4], pv[5]), pack_f16x2(pv[6], pv[7])};
    }
    l_run += rs;
    // the next tile's upcast (independent of this P.V) in the same block as the MFMAs
    constexpr int Q = 1 - decltype(P)::value;
    if (conv_next) convert_chunks(Int<Q>{});
    int v_lo, v_hi;
    v_bases(v_lo, v_hi);
#pragma unroll
    for (int mt = 0; mt < kMW; ++mt) {
      const int col = 32 * (kMW * half + mt);
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const u32x2 lo = lds_read_tr16(F + v_lo + 16 * kk * kKS + col);
        const u32x2 hi = lds_read_tr16(F + v_hi + 16 * kk * kKS + col);
        acc[mt] = mfma32x32x16_f16(u32x4{lo.x, lo.y, hi.x, hi.y}, pb[kk], acc[mt]);
      }
    }
  };

  // ---- pipeline.  Step t computes tile t from fp16 buffer t&1 and upcasts tile t+1 into
  // the other buffer; steps alternate the parity at compile time so the compiler can tell
  // the raw buffers apart.  Barrier 1 (step start): step t-1 is done everywhere, so fp16
  // buffer (t+1)&1, raw buffer t&1 and the S exchange are free.  Barrier 2 (LDS only --
  // a later DMA may stay in flight) publishes the S shares of split waves.  Each wave
  // waits for its own share of tile t+1's DMA before the barrier that precedes the
  // upcast; tile t+2's DMA goes out into raw buffer t&1 after that upcast's inputs are
  // safe.
  //   early upcast: wait, barrier 1, upcast t+1, S, issue t+2, barrier 2, softmax, P.V
  //   late upcast:  barrier 1, S, wait, barrier 2, issue t+2, softmax, P.V with upcast t+1
  const int n_tiles = (n_keys + kKT - 1) / kKT;
  auto publish = [&](const f32x16& s) {
    if constexpr (SPLIT > 1) {
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        f32x4* xo = x_own();
        xo[64 * i4] = f32x4{s[4 * i4], s[4 * i4 + 1], s[4 * i4 + 2], s[4 * i4 + 3]};
      }
    }
  };
  auto step = [&](auto P, int t) {
    constexpr int Q = 1 - decltype(P)::value;
    const bool conv = t + 1 < n_tiles;
    if constexpr (LATE_CONV) {
      __syncthreads();
      const f32x16 s = qk(P);
      publish(s);
      wait_vm0();
      barrier_lds();
      if (t + 2 < n_tiles) issue(P, t + 2);
      softmax_pv(P, s, t, conv);
      if (conv) convert_meta(Int<Q>{});
    } else {
      wait_vm0();
      __syncthreads();
      if (conv) convert(Int<Q>{});
      const f32x16 s = qk(P);
      if (t + 2 < n_tiles) issue(P, t + 2);
      publish(s);
      if constexpr (SPLIT > 1) barrier_lds();
      softmax_pv(P, s, t, false);
    }
  };
  issue(Int<0>{}, 0);
  wait_vm0();
  __syncthreads();
  convert(Int<0>{});
  if (n_tiles > 1) issue(Int<1>{}, 1);
  for (int t = 0; t < n_tiles; t += 2) {
    step(Int<0>{}, t);
    if (t + 1 < n_tiles) step(Int<1>{}, t + 1);
  }

  // ---- finish: full row sum over the two lane halves, write this wave's dims
  const float l_tot = halves_sum(l_run);
  if (!row_ok) return;
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const float lse2 = l_tot > 0.f ? m_run + __log2f(l_tot) : -INFINITY;
  // acc[mt][4q + i] = O[row][32 (kMW half + mt) + 8q + 4h + i]
  if constexpr (SPARSE) {
    uint16_t* op = sa.out + ((size_t)unit * Hq + row) * kDv + 32 * kMW * half + 4 * h;
#pragma unroll
    for (int mt = 0; mt < kMW; ++mt)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        u32x2 w;
        w.x = pack_bf16x2(acc[mt][4 * q] * inv, acc[mt][4 * q + 1] * inv);
        w.y = pack_bf16x2(acc[mt][4 * q + 2] * inv, acc[mt][4 * q + 3] * inv);
        *reinterpret_cast<u32x2*>(op + 32 * mt + 8 * q) = w;
      }
    if (sa.lse != nullptr && h == 0 && half == 0)
      sa.lse[(size_t)unit * Hq + row] = lse2 == -INFINITY ? -INFINITY : lse2 * kLn2;
  } else {
    const size_t pbase = ((size_t)unit * da.max_splits + unit_split) * rows_total + row;
    float* op = da.part_o + pbase * kDv + 32 * kMW * half + 4 * h;
#pragma unroll
    for (int mt = 0; mt < kMW; ++mt)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<f32x4*>(op + 32 * mt + 8 * q) =
            f32x4{acc[mt][4 * q], acc[mt][4 * q + 1], acc[mt][4 * q + 2], acc[mt][4 * q + 3]} * inv;
    if (h == 0 && half == 0) da.part_lse[pbase] = lse2;
  }
}

#ifndef PA_MLA_DECODE_WAVES
#define PA_MLA_DECODE_WAVES 8
#endif
#ifndef PA_MLA_DECODE_SPLIT
#define PA_MLA_DECODE_SPLIT 2
#endif
constexpr int kDecodeWaves = PA_MLA_DECODE_WAVES, kDecodeSplit = PA_MLA_DECODE_SPLIT;
#ifndef PA_MLA_SPARSE_WAVES
#define PA_MLA_SPARSE_WAVES 8
#endif
#ifndef PA_MLA_SPARSE_SPLIT
#define PA_MLA_SPARSE_SPLIT 4
#endif
constexpr int kSparseWaves = PA_MLA_SPARSE_WAVES, kSparseSplit = PA_MLA_SPARSE_SPLIT;
#ifndef PA_MLA_SPARSE_STAGE
#define PA_MLA_SPARSE_STAGE 1
#endif
constexpr bool kSparseStage = PA_MLA_SPARSE_STAGE != 0;   // selections and block ids staged in LDS
constexpr int kDecodeRows = 32 * kDecodeWaves / kDecodeSplit, kSparseRows = 32 * kSparseWaves / kSparseSplit;

}  // namespace

template <bool REDO>
static hipError_t mla_decode_launch(const MlaDecodeArgs& a, hipStream_t stream) {
  const int rows = a.q_per_seq * a.num_q_heads;
  const unsigned grid = (unsigned)a.num_seqs * a.max_splits * ((rows + kDecodeRows - 1) / kDecodeRows);
  if (grid == 0) return hipSuccess;
  SparseMlaArgs none{};
  hipLaunchKernelGGL((mla_kernel<false, kDecodeWaves, kDecodeSplit, true, false, REDO>), dim3(grid),
                     dim3(64 * kDecodeWaves), 0, stream, a, none);
  return hipGetLastError();
}
hipError_t launch_mla_decode_exact(const MlaDecodeArgs& a, hipStream_t stream) { return mla_decode_launch<true>(a, stream); }

template <bool REDO>
static hipError_t sparse_mla_launch(const SparseMlaArgs& a, hipStream_t stream) {
  const unsigned grid = (unsigned)a.n_q * ((a.num_q_heads + kSparseRows - 1) / kSparseRows);
  if (grid == 0) return hipSuccess;
  MlaDecodeArgs none{};
  if constexpr (kSparseStage) {
    if (a.k <= kSelLds) {
      hipLaunchKernelGGL((mla_kernel<true, kSparseWaves, kSparseSplit, true, true, REDO>), dim3(grid),
                         dim3(64 * kSparseWaves), 0, stream, none, a);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((mla_kernel<true, kSparseWaves, kSparseSplit, false, true, REDO>), dim3(grid),
                     dim3(64 * kSparseWaves), 0, stream, none, a);
  return hipGetLastError();
}
hipError_t launch_sparse_mla_exact(const SparseMlaArgs& a, hipStream_t stream) { return sparse_mla_launch<true>(a, stream); }

}  // namespace pa
