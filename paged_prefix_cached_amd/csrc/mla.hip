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
// latent + 64 rope) and d_v = 512 (the latent itself).  A workgroup holds NP wave pairs;
// pair p owns 32 query rows and every pair reads the same keys (decode: 4 pairs = 128
// rows, e.g. two MTP tokens x 64 heads; sparse: 2 pairs = the 64 heads of one query).
// Keys go in 32-key tiles through a three-stage pipeline:
//   1. LDS-DMA (global_load_lds, 16 bytes a lane) gathers tile t+2's FP8 rows through the
//      block table into a raw LDS buffer -- no registers held while the loads fly.  Block
//      ids (decode: the split's range; sparse: the sequence's row) and, for sparse, the
//      selected positions are staged in LDS once.
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

#ifndef PA_MLA_DECODE_PAIRS
#define PA_MLA_DECODE_PAIRS 4
#endif

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kDqk = 576, kDv = 512, kBs = 64;
constexpr int kKT = 32;                   // keys per tile
constexpr int kKS = 608;                  // fp16 per LDS row: 1,216 B, 304 dwords = 48 mod 64
constexpr int kQH = kDqk / 32;            // 18 QK k-steps of 16 per wave (half of 576)
constexpr int kMH = kDv / 64;             // 8 O^T tiles of 32 dims per wave (half of 512)
constexpr int kChunks = kKT * (kDqk / 16);   // 16-byte FP8 chunks per tile (1,152)
constexpr int kWaveLoads = kChunks / 64;     // 1 KB DMA wave-loads per tile (18)
constexpr int kBtLds = 4096;              // block-table entries staged in LDS (sparse)
constexpr int kSelLds = 2048;             // selected positions staged in LDS (sparse)
static_assert(kChunks % 64 == 0, "tile is a whole number of wave-loads");

template <int N>
using Int = std::integral_constant<int, N>;

__device__ __forceinline__ void dma16(const void* src, void* lds_dst) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds_dst, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void* src, void* lds_dst) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds_dst, 4, 0, 0);
}
// Wait until at most N vector-memory operations of this wave are outstanding (gfx9
// s_waitcnt encoding; expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

template <bool SPARSE, int NP>
__global__ __launch_bounds__(NP * 128, 1) void mla_kernel(MlaDecodeArgs da, SparseMlaArgs sa) {
  constexpr int NW = 2 * NP, NT = NW * 64;
  // DMA operations per wave per tile: wave-loads w, w + NW, ...; the last wave also
  // fetches the 32 scales.  MIN_OPS is the fewest any wave issues.
  constexpr int MIN_OPS = kWaveLoads / NW;
  static_assert(MIN_OPS >= 1 && MIN_OPS < 64, "DMA accounting");
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
  __shared__ __attribute__((aligned(16))) f32x4 xs[NW * 4 * 64]; // partial S exchange
  __shared__ int32_t bt_s[SPARSE ? kBtLds : kDecodeSplitMla / kBs + 1];
  __shared__ int32_t sel_s[SPARSE ? kSelLds : 1];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, h = lane >> 5;
  const int pair = wave >> 1, half = wave & 1;

  // ---- work unit
  const uint16_t* qbase;
  const int32_t* bt_row;
  const int32_t* sel_g = nullptr;
  const uint8_t* kv;
  const float* kv_scale;
  int Hq, n_keys, k_begin = 0, n_lblocks, L = 0, T = 1, row0, unit = 0, unit_split = 0;
  int lb_base = 0, n_bt, num_blocks;
  bool bt_in_lds = true, sel_in_lds = true;
  float scale_log2;
  if constexpr (SPARSE) {
    Hq = sa.num_q_heads;
    const int rblocks = (Hq + 32 * NP - 1) / (32 * NP);
    const int i = blockIdx.x / rblocks;
    row0 = (blockIdx.x % rblocks) * 32 * NP;
    unit = i;
    qbase = sa.q + (size_t)i * Hq * kDqk;
    kv = sa.kv; kv_scale = sa.kv_scale; num_blocks = sa.num_blocks;
    bt_row = sa.bt + (size_t)sa.q_seq[i] * sa.bt_stride;
    sel_g = sa.topk + (size_t)i * sa.k;
    n_keys = sa.k;
    n_lblocks = sa.bt_stride;
    bt_in_lds = sa.bt_stride <= kBtLds;
    sel_in_lds = sa.k <= kSelLds;
    n_bt = bt_in_lds ? sa.bt_stride : 0;
    scale_log2 = sa.scale_log2;
  } else {
    Hq = da.num_q_heads;
    T = da.q_per_seq;
    const int rows = T * Hq;
    const int rblocks = (rows + 32 * NP - 1) / (32 * NP);
    const int n_units = da.num_seqs * da.max_splits * rblocks;
    const int logical = xcd_swizzle(blockIdx.x, n_units);
    const int rb = logical % rblocks;
    unit_split = (logical / rblocks) % da.max_splits;
    unit = logical / (rblocks * da.max_splits);
    row0 = rb * 32 * NP;
    L = min(da.context_len[unit], da.max_context_len);
    k_begin = unit_split * kDecodeSplitMla;
    if (k_begin >= L) return;                         // uniform for the workgroup
    n_keys = min(L - k_begin, kDecodeSplitMla);
    qbase = da.q + (size_t)unit * rows * kDqk;
    kv = da.kv; kv_scale = da.kv_scale; num_blocks = da.num_blocks;
    bt_row = da.bt + (size_t)unit * da.bt_stride;
    n_lblocks = (L + kBs - 1) / kBs;
    lb_base = k_begin / kBs;
    n_bt = (k_begin + n_keys + kBs - 1) / kBs - lb_base;   // <= kDecodeSplitMla / kBs
    scale_log2 = da.scale_log2;
  }
  const int rows_total = SPARSE ? Hq : T * Hq;

  // ---- this lane's query row (C column = lane % 32) and its half of the fp16 Q
  const int row = row0 + pair * 32 + l32;
  const bool row_ok = row < rows_total;
  const int row_c = row_ok ? row : rows_total - 1;
  const int pos = SPARSE ? 0x7fffffff : (L - T + row_c / Hq);
  u32x4 qb[kQH];
  {
    const uint16_t* qp = qbase + (size_t)row_c * kDqk + 288 * half + 8 * h;
#pragma unroll
    for (int ks = 0; ks < kQH; ++ks) {
      const u32x4 v = ld16(qp + 16 * ks);
      qb[ks] = u32x4{bf16x2_to_f16x2(v.x), bf16x2_to_f16x2(v.y), bf16x2_to_f16x2(v.z), bf16x2_to_f16x2(v.w)};
    }
  }

  // ---- stage validated block ids and, for sparse, the selected positions
  for (int j = tid; j < n_bt; j += NT) bt_s[j] = phys_block(bt_row, lb_base + j, n_lblocks, num_blocks);
  if constexpr (SPARSE) {
    if (sel_in_lds)
      for (int j = tid; j < n_keys; j += NT) sel_s[j] = sel_g[j];
  }
  __syncthreads();
  // j-th key of the unit -> physical block (or -1) and its logical position
  auto key_loc = [&](int j, int& idx) -> int {
    idx = -1;
    if (j >= n_keys) return -1;
    if constexpr (SPARSE) {
      idx = sel_in_lds ? sel_s[j] : sel_g[j];
      if (idx < 0) return -1;
      const int lb = idx / kBs;
      if (bt_in_lds) return lb < n_bt ? bt_s[lb] : -1;
      return phys_block(bt_row, lb, n_lblocks, num_blocks);
    } else {
      idx = k_begin + j;
      return bt_s[idx / kBs - lb_base];
    }
  };

  // ---- stage 1: DMA tile tt into raw buffer P
  auto issue = [&](auto P, int tt) {
    uint8_t* R = P ? r1 : r0;
    float* RS = P ? rs1 : rs0;
    int32_t* RK = P ? rk1 : rk0;
    const int kb = tt * kKT;
    int ln = lane;
    asm volatile("" : "+v"(ln));   // recompute the lane's indices here, keep no VGPRs for them
    for (int j = wave; j < kWaveLoads; j += NW) {
      const int c = 64 * j + ln;
      const int key = c / (kDqk / 16), dc = c % (kDqk / 16);
      int idx;
      const int pb = key_loc(kb + key, idx);
      // invalid keys read a harmless in-bounds row; stage 2 replaces them by zeros
      const uint8_t* src = pb >= 0 ? kv + ((size_t)pb * kBs + idx % kBs) * kDqk + 16 * dc : kv;
      dma16(src, R + 1024 * j);
    }
    if (wave == NW - 1 && ln < kKT) {
      int idx;
      const int pb = key_loc(kb + ln, idx);
      dma4(pb >= 0 ? kv_scale + (size_t)pb * kBs + idx % kBs : kv_scale, RS);
      RK[ln] = pb >= 0 ? idx : -1;
    }
  };
  // ---- stage 2: raw buffer P -> fp16 tile P (and its key metadata)
  auto convert = [&](auto P) {
    const uint8_t* R = P ? r1 : r0;
    const float* RS = P ? rs1 : rs0;
    const int32_t* RK = P ? rk1 : rk0;
    uint16_t* F = fb[P];
    int th = tid;
    asm volatile("" : "+v"(th));
    for (int c = th; c < kChunks; c += NT) {
      const int key = c / (kDqk / 16), dc = c % (kDqk / 16);
      const int v = (key >> 2) & 3;
      u32x4 lo = {0, 0, 0, 0}, hi = {0, 0, 0, 0};
      if (RK[key] >= 0) {
        const u32x4 raw = *reinterpret_cast<const u32x4*>(R + 16 * c);
        const u32x2 a0 = fp8x4_to_f16x4(raw.x), a1 = fp8x4_to_f16x4(raw.y);
        const u32x2 a2 = fp8x4_to_f16x4(raw.z), a3 = fp8x4_to_f16x4(raw.w);
        lo = u32x4{a0.x, a0.y, a1.x, a1.y};
        hi = u32x4{a2.x, a2.y, a3.x, a3.y};
      }
      uint16_t* rp = F + key * kKS;
      st16(rp + 8 * ((2 * dc) ^ v), lo);
      st16(rp + 8 * ((2 * dc + 1) ^ v), hi);
    }
    if (th < kKT) {
      const int id = RK[th];
      const float sc = RS[th];
      fk[P][th] = id;
      fks[P][th] = id >= 0 ? sc * scale_log2 : 0.f;
      fvs[P][th] = id >= 0 ? sc : 0.f;
    }
  };

  // ---- per-lane LDS offsets (fp16 units) into an fp16 tile, swizzle folded in.
  // K fragment of k-step ks (global 0..35): key row l32, logical chunk 2ks + h stored at
  // chunk (2ks + h) ^ v, v = (l32 / 4) & 3; ks parity decides the sign of the v/2 term.
  const int vk = (l32 >> 2) & 3;
  const int k_even = l32 * kKS + 8 * (h ^ (vk & 1)) + 16 * (vk >> 1);
  const int k_odd = l32 * kKS + 8 * (h ^ (vk & 1)) - 16 * (vk >> 1);
  // V^T fragments of k-step kk and output tile mt: rows 16kk + 4h + n/4 (first read) and
  // 8 rows further (second), logical chunk 4mt + 2(g%2) + (n%4)/2, fp16 offset 4(n&1).
  const int g = lane >> 4, n = lane & 15;
  const int vrow = 4 * h + (n >> 2);
  const int vsub = 2 * (g & 1) + ((n & 3) >> 1);
  const int v_lo = vrow * kKS + 8 * (vsub ^ h) + 4 * (n & 1);
  const int v_hi = (vrow + 8) * kKS + 8 * (vsub ^ ((h + 2) & 3)) + 4 * (n & 1);

  f32x16 acc[kMH];
#pragma unroll
  for (int mt = 0; mt < kMH; ++mt)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[mt][i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  f32x4* x_own = xs + wave * 256 + lane;
  const f32x4* x_pair = xs + (wave & ~1) * 256 + lane;   // half 0's partial, then half 1's

  // ---- stage 3, first half: partial S^T over this wave's 288 dims, published to the peer
  auto qk_partial = [&](auto P) -> void {
    const uint16_t* F = fb[P];
    f32x16 s;
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = 0.f;
#pragma unroll
    for (int k = 0; k < kQH; ++k) {
      const int ks = kQH * half + k;             // parity of ks equals parity of k
      const uint16_t* kp = F + ((k & 1) ? k_odd : k_even) + 16 * ks;
      s = mfma32x32x16_f16(*reinterpret_cast<const u32x4*>(kp), qb[k], s);
      if (k % 3 == 2) __builtin_amdgcn_sched_barrier(0);   // bound the read lookahead
    }
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) x_own[64 * i4] = f32x4{s[4 * i4], s[4 * i4 + 1], s[4 * i4 + 2], s[4 * i4 + 3]};
  };
  // ---- stage 3, second half: full S, online softmax, O^T += V^T P^T for this wave's dims
  auto softmax_pv = [&](auto P) {
    const uint16_t* F = fb[P];
    // full S = half 0 + half 1, the same operation in both waves of the pair
    f32x16 s;
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const f32x4 a = x_pair[64 * i4], b = x_pair[256 + 64 * i4];
#pragma unroll
      for (int i = 0; i < 4; ++i) s[4 * i4 + i] = a[i] + b[i];
    }
    // scale, mask, running maximum; lane holds row `row`, keys 8(i/4) + 4h + i%4
    float mx = -INFINITY;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int kb4 = 8 * q4 + 4 * h;
      const int4 id = *reinterpret_cast<const int4*>(&fk[P][kb4]);
      const f32x4 ksc = *reinterpret_cast<const f32x4*>(&fks[P][kb4]);
      const int idv[4] = {id.x, id.y, id.z, id.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float v = (idv[i] >= 0 && idv[i] <= pos) ? s[4 * q4 + i] * ksc[i] : -INFINITY;
        s[4 * q4 + i] = v;
        mx = fmaxf(mx, v);
      }
      __builtin_amdgcn_sched_barrier(0);   // one group of key metadata in registers at a time
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    if (__ballot(m_new > m_run) != 0) {
      const float alpha = m_run == -INFINITY ? 0.f : fast_exp2(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int mt = 0; mt < kMH; ++mt) acc[mt] *= alpha;
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
#pragma unroll
    for (int mt = 0; mt < kMH; ++mt) {
      const int col = 32 * (kMH * half + mt);
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const u32x2 lo = lds_read_tr16(F + v_lo + 16 * kk * kKS + col);
        const u32x2 hi = lds_read_tr16(F + v_hi + 16 * kk * kKS + col);
        acc[mt] = mfma32x32x16_f16(u32x4{lo.x, lo.y, hi.x, hi.y}, pb[kk], acc[mt]);
      }
      if (mt % 2 == 1) __builtin_amdgcn_sched_barrier(0);
    }
  };

  const int n_tiles = (n_keys + kKT - 1) / kKT;
  // One pipeline step on tile t, whose fp16 tile is buffer P.  On entry tile t+1's DMA
  // (raw buffer !P) is in flight and raw buffer P is free.  Steps alternate P at compile
  // time so the compiler can tell the raw buffers apart.
  auto step = [&](auto P, int t) {
    constexpr int Q = 1 - decltype(P)::value;
    const bool more2 = t + 2 < n_tiles;
    if (more2) issue(P, t + 2);
    qk_partial(P);
    // tile t+1's raw bytes: this wave's DMAs done (only tile t+2's may remain) ...
    if (more2) wait_vm<MIN_OPS>(); else wait_vm<0>();
    __syncthreads();                                   // ... and everyone's; S partials published
    softmax_pv(P);
    if (t + 1 < n_tiles) convert(Int<Q>{});
    __syncthreads();                                   // fp16 tile t+1 ready; X and buffers free
  };

  issue(Int<0>{}, 0);
  if (n_tiles > 1) {
    issue(Int<1>{}, 1);
    wait_vm<MIN_OPS>();
  } else {
    wait_vm<0>();
  }
  __syncthreads();
  convert(Int<0>{});
  __syncthreads();
  for (int t = 0; t < n_tiles; t += 2) {
    step(Int<0>{}, t);
    if (t + 1 < n_tiles) step(Int<1>{}, t + 1);
  }

  // ---- finish: full row sum over the two lane halves, write this wave's 256 dims
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (!row_ok) return;
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const float lse2 = l_tot > 0.f ? m_run + __log2f(l_tot) : -INFINITY;
  // acc[mt][4q + i] = O[row][256 half + 32mt + 8q + 4h + i]
  if constexpr (SPARSE) {
    uint16_t* op = sa.out + ((size_t)unit * Hq + row) * kDv + 256 * half + 4 * h;
#pragma unroll
    for (int mt = 0; mt < kMH; ++mt)
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
    float* op = da.part_o + pbase * kDv + 256 * half + 4 * h;
#pragma unroll
    for (int mt = 0; mt < kMH; ++mt)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<f32x4*>(op + 32 * mt + 8 * q) =
            f32x4{acc[mt][4 * q], acc[mt][4 * q + 1], acc[mt][4 * q + 2], acc[mt][4 * q + 3]} * inv;
    if (h == 0 && half == 0) da.part_lse[pbase] = lse2;
  }
}

constexpr int kDecodePairs = PA_MLA_DECODE_PAIRS, kSparsePairs = 2;

}  // namespace

hipError_t launch_mla_decode(const MlaDecodeArgs& a, hipStream_t stream) {
  const int rows = a.q_per_seq * a.num_q_heads;
  const unsigned grid = (unsigned)a.num_seqs * a.max_splits * ((rows + 32 * kDecodePairs - 1) / (32 * kDecodePairs));
  if (grid == 0) return hipSuccess;
  SparseMlaArgs none{};
  hipLaunchKernelGGL((mla_kernel<false, kDecodePairs>), dim3(grid), dim3(128 * kDecodePairs), 0, stream, a, none);
  return hipGetLastError();
}

hipError_t launch_sparse_mla(const SparseMlaArgs& a, hipStream_t stream) {
  const unsigned grid = (unsigned)a.n_q * ((a.num_q_heads + 32 * kSparsePairs - 1) / (32 * kSparsePairs));
  if (grid == 0) return hipSuccess;
  MlaDecodeArgs none{};
  hipLaunchKernelGGL((mla_kernel<true, kSparsePairs>), dim3(grid), dim3(128 * kSparsePairs), 0, stream, none, a);
  return hipGetLastError();
}

}  // namespace pa
