// Paged GQA decode (bf16 K/V, block size 16) that reads every distinct KV block once per
// group of sequences and spreads the work evenly over the GPU.
//
// Sources: vLLM AgentX article (news.ainew.jp), "Re-evaluating agentic workloads" (>96 %
// prefix-cache hits; sub-agents fork from the parent context, so sequences in flight share
// long prefixes), "Hybrid KV cache management" (one shared block pool: shared prefixes are
// the same physical blocks, Figure 4) and "Kimi K3" (partial outputs and their
// log-sum-exp merged with online softmax, Figure 7).
//
// A group holds M = 32 / (T*G) consecutive sequences, so its T query tokens x G heads per
// sequence fill the 32 rows of a v_mfma_f32_32x32x16 tile (8 sequences x 4 heads for
// 32q/8kv heads and one token).  Three launches (four past the LDS index):
//   1. decode_plan_kernel lists, for every group and 32-key tile (two 16-token blocks),
//      the DISTINCT block pairs its members reference, each with the set of members that
//      share it and the number of its keys that hold data.  Blocks that forked sequences
//      share become one pass for all of them: fetched from HBM once, not once per member.
//   2. The passes of all groups are numbered consecutively (region by region) and cut into
//      pieces at the attention grid's workgroup boundaries: by every attention workgroup
//      itself, in LDS, or -- when the region and piece starts exceed its LDS index -- by a
//      separate decode_scan_kernel into the workspace.
//   3. gqa_decode_kernel: one workgroup per compute unit, each taking an equal share of
//      the pass list -- every pass costs the same (two blocks of K and V per KV head), so
//      the shares finish together -- with one wave per KV head, so the eight waves read
//      the same blocks for all heads and never wait for one another.  Each piece (a
//      group's passes inside one workgroup's share) yields a normalised partial output
//      and log2-sum-exp per head.
//   4. combine_kernel merges each row's partials in pass order.
// Every partition depends on the inputs only, so results are identical run to run.
#include <algorithm>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

GqaDecodeDims gqa_decode_dims(int num_seqs, int q_per_seq, int num_q_heads, int num_kv_heads,
                              int max_context_len) {
  GqaDecodeDims d{};
  const int R = q_per_seq * (num_q_heads / num_kv_heads);
  d.members = R >= 32 ? 1 : 32 / R;
  d.n_groups = (num_seqs + d.members - 1) / d.members;
  const long n_tiles = (max_context_len + 31) / 32;
  d.n_chunks = (int)((n_tiles + kPlanTiles - 1) / kPlanTiles);
  d.region_cap = kPlanTiles * d.members;
  d.grid = device_cus();
  d.subs = (num_kv_heads < 8 && 8 % num_kv_heads == 0) ? 8 / num_kv_heads : 1;
  // pieces: every group's passes cut at the workgroup boundaries
  d.pieces_cap = d.n_groups + d.grid - 1;
  d.scan_in_kernel = (long)d.n_groups * d.n_chunks + d.n_groups + 2 <= kDecodeIdxLds;
  return d;
}

namespace {

// Waves per attention workgroup (one workgroup per compute unit, two waves per SIMD): one
// per KV head of the 8, or 8 / Hkv sub-ranges per head for fewer heads.
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kTile = 32;               // keys per pass (two 16-token blocks)

// ---------------------------------------------------------------------------------
// 1. Plan: one workgroup per (group, chunk of kPlanTiles tiles), one thread per tile.
// Member m takes part in tile t iff 32t < L_m; its pair is (block 2t, block 2t+1), each
// -1 when past its blocks or out of range (read as zeros).  Pairs are deduplicated in
// member order; a pass lists the members sharing its pair and how many of its 32 keys
// hold data for the longest of them.
__global__ __launch_bounds__(256) void decode_plan_kernel(GqaDecodeArgs a) {
  __shared__ int2 pr[32][kPlanTiles];
  __shared__ int len_s[32];
  __shared__ int wsum[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int M = a.dims.members, region = blockIdx.x;
  const int g = region / a.dims.n_chunks, c = region % a.dims.n_chunks;
  const int s0 = g * M;
  if (tid < 32) {
    int L = 0;
    if (tid < M && s0 + tid < a.num_seqs) L = min(max(a.context_len[s0 + tid], 0), a.max_context_len);
    len_s[tid] = L;                     // read after the scan's barrier below
  }
  const int tile = c * kPlanTiles + tid, kb = tile * kTile;
  const int ia = min(2 * tile, a.bt_stride - 1), ib = min(2 * tile + 1, a.bt_stride - 1);
  uint32_t part = 0;                    // members taking part in this tile
  for (int m0 = 0; m0 < M; m0 += 8) {   // 8 members' loads in flight at a time
    int ra[8], rb[8], Lm[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      // The lengths and the table entries load together: the entries come from an existing
      // row at clamped columns, so they stay in bounds whatever the lengths turn out to be,
      // and only those inside the member's blocks are used.
      const int mm = m0 + i;
      const bool real = mm < M && s0 + mm < a.num_seqs;
      Lm[i] = real ? min(max(a.context_len[s0 + mm], 0), a.max_context_len) : 0;
      const int32_t* row = a.bt + (size_t)min(s0 + mm, a.num_seqs - 1) * a.bt_stride;
      ra[i] = row[ia];
      rb[i] = row[ib];
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (m0 + i >= M) break;
      const bool ok = kb < Lm[i];
      const int nl = ok ? (Lm[i] + 15) >> 4 : 0;
      if (ok) part |= 1u << (m0 + i);
      int2 p = {-1, -1};
      if (2 * tile < nl && ra[i] >= 0 && ra[i] < a.num_blocks) p.x = ra[i];
      if (2 * tile + 1 < nl && rb[i] >= 0 && rb[i] < a.num_blocks) p.y = rb[i];
      pr[m0 + i][tid] = p;
    }
  }
  // first occurrences of each distinct pair (a column of pr is this thread's alone)
  uint32_t first = 0;
  for (int mm = 0; mm < M; ++mm) {
    if (!((part >> mm) & 1)) continue;
    const int2 p = pr[mm][tid];
    bool is_first = true;
    for (int m2 = 0; m2 < mm; ++m2) {
      const int2 q2 = pr[m2][tid];
      if (((part >> m2) & 1) && q2.x == p.x && q2.y == p.y) { is_first = false; break; }
    }
    if (is_first) first |= 1u << mm;
  }
  const int cnt = __builtin_popcount(first);
  // exclusive scan of cnt over the workgroup
  int x = cnt;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  int off = x - cnt, total = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    off += w < wave ? wsum[w] : 0;
    total += wsum[w];
  }
  if (tid == 0) a.n_passes[region] = total;
  uint32_t* out = a.passes + ((size_t)region * a.dims.region_cap + off) * 4;
  for (int mm = 0; mm < M; ++mm) {
    if (!((first >> mm) & 1)) continue;
    const int2 p = pr[mm][tid];
    uint32_t mask = 0;
    int Lp = 0;
    for (int m2 = mm; m2 < M; ++m2) {
      const int2 q2 = pr[m2][tid];
      if (((part >> m2) & 1) && q2.x == p.x && q2.y == p.y) {
        mask |= 1u << m2;
        Lp = max(Lp, len_s[m2]);
      }
    }
    const int nvalid = min(kTile, Lp - kb);   // >= 1: every member here has L > kb
    st16(out, u32x4{(uint32_t)(kb | (nvalid - 1)), (uint32_t)p.x, (uint32_t)p.y, mask});
    out += 4;
  }
}

// ---------------------------------------------------------------------------------
// 2. Numbering (by every attention workgroup in its LDS, or past the LDS index by
// decode_scan_kernel, one workgroup): region_start[r] = passes of the regions before r in region order
// (the compact pass numbering; region_start[R] = P, the total), and piece_start[g] = pieces
// before group g.  A group's regions are consecutive, so its passes are one contiguous
// range of the numbering.  The attention grid splits [0, P) over N = min(grid, P)
// workgroups, never into an empty range (P / N >= 1).  A piece is a group's share of one
// workgroup's range, so group g holds wg_of(last) - wg_of(first) + 1 pieces (0 when it has
// no pass), numbered consecutively in pass order: a workgroup's range that crosses a
// region boundary inside one group stays one piece.
// Workgroup w of N takes passes [wg_bound(w), wg_bound(w + 1)).  Workgroups go to the 8
// XCDs round robin (XCD = w mod 8), and the odd XCDs run the same passes about 4.5 % slower
// (per-workgroup end stamps on MI355X, repeatable launch to launch); so when every
// workgroup has plenty of passes the even ones take kXcdSkew / 1024 more than an equal share
// and the odd ones as much less.
constexpr long kXcdSkew = 23;
__device__ __forceinline__ long wg_bound(long w, long P, long N) {
  if (P < 8 * N) return w * P / N;                  // few passes: equal shares
  // weights 1024 +- kXcdSkew alternate, so the cumulative weight is 1024 w + kXcdSkew (w & 1)
  return P * (1024 * w + kXcdSkew * (w & 1)) / (1024 * N + kXcdSkew * (N & 1));
}
// wg_of(x): the workgroup whose range holds pass x, max{w : wg_bound(w) <= x}.  The skew
// moves a boundary by less than one share, so the equal-share estimate is off by at most one.
__device__ __forceinline__ int wg_of(long x, long P, long N) {
  long w = ((x + 1) * N - 1) / P;
  w = w < 0 ? 0 : (w > N - 1 ? N - 1 : w);
  while (w + 1 < N && wg_bound(w + 1, P, N) <= x) ++w;
  while (w > 0 && wg_bound(w, P, N) > x) --w;
  return (int)w;
}
__device__ __forceinline__ long active_wgs(long grid, long P) { return grid < P ? grid : P; }

// The region holding pass x: the first r in [0, n) with rs[r + 1] > x (one exists, since
// rs[n] = P > x).  A wave tests 64 evenly spaced candidates per round (one load per lane),
// so the search costs one or two dependent loads rather than log2(n).
__device__ __forceinline__ int region_of(const int32_t* rs, int n, int x) {
  const int lane = threadIdx.x & 63;
  int r0 = 0, r1 = n - 1;                           // the answer lies in [r0, r1]
  while (r0 < r1) {
    const int span = r1 - r0 + 1, step = (span + 63) / 64;
    const int r = r0 + lane * step;
    const bool past = r <= r1 && rs[r + 1] > x;
    const uint64_t bal = __ballot(past);
    if (bal == 0) {                                 // the answer follows the last candidate
      r0 += ((span - 1) / step) * step + 1;
    } else {
      const int L = __builtin_ctzll(bal);
      r1 = r0 + L * step;
      r0 = L == 0 ? r0 : r0 + (L - 1) * step + 1;
    }
  }
  return r0;
}

// Exclusive prefix sum over a workgroup of NW waves; *total = the sum over all threads.
template <int NW>
__device__ __forceinline__ int block_exclusive_scan(int v, int* wsum, int* total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  int off = x - v, t = 0;
  for (int w = 0; w < NW; ++w) {
    off += w < wave ? wsum[w] : 0;
    t += wsum[w];
  }
  __syncthreads();
  *total = t;
  return off;
}

__global__ __launch_bounds__(1024) void decode_scan_kernel(GqaDecodeArgs a) {
  __shared__ int wsum[16];
  const int tid = threadIdx.x;
  const int n = a.dims.n_groups * a.dims.n_chunks;
  int running = 0;
  for (int base = 0; base < n; base += 1024) {
    const int r = base + tid;
    int total;
    const int off = block_exclusive_scan<16>(r < n ? a.n_passes[r] : 0, wsum, &total);
    if (r < n) a.region_start[r] = running + off;
    running += total;
  }
  if (tid == 0) a.region_start[n] = running;
  __syncthreads();
  const long P = running, N = active_wgs(a.dims.grid, P);
  const int NG = a.dims.n_groups, NC = a.dims.n_chunks;
  int pieces = 0;
  for (int base = 0; base < NG; base += 1024) {
    const int g = base + tid;
    int cnt = 0;
    if (g < NG) {
      const int s0 = a.region_start[g * NC], s1 = a.region_start[(g + 1) * NC];
      cnt = s1 > s0 ? wg_of(s1 - 1, P, N) - wg_of(s0, P, N) + 1 : 0;
    }
    int total;
    const int off = block_exclusive_scan<16>(cnt, wsum, &total);
    if (g < NG) a.piece_start[g] = pieces + off;
    pieces += total;
  }
  if (tid == 0) a.piece_start[NG] = pieces;
}

// ---------------------------------------------------------------------------------
// 3. Attention: workgroup w of N = min(grid, P) takes the passes [wg_bound(w), wg_bound(w + 1))
// of the compact pass list -- equal shares up to the XCD skew, so the workgroups finish
// together -- and walks them group by group (a piece per group it meets; inside a group a
// cursor over the region starts finds each pass's slot in the plan).  Each wave takes one KV
// head (and, when the heads are fewer than 8 and divide 8, one of 8 / Hkv equal
// sub-ranges of the piece), so the 8 waves of a workgroup read the same blocks for all
// heads at once (a block's K, or V, is Hkv * 4 KB contiguous) and never wait for one
// another: there is no barrier and no merge across waves.  Per pass a wave
//   * has issued the pass's K and V loads while the previous pass was computed
//     (register double buffering), and its descriptor one pass earlier still;
//   * uses K straight from registers as the A operand of S^T = K Q^T; the Q^T fragments
//     (B operand, lane = query row) come from the wave's own LDS copy of its 32 rows;
//   * masks rows whose member does not share the pass and keys past each row's
//     position, then updates its online softmax in-lane (one xor-32 step per row);
//   * writes V (bf16; keys without data zeroed) row-major into its own LDS slice and
//     accumulates O^T += V^T P^T with two v_mfma_f32_32x32x16_bf16, P split into bf16
//     hi + lo parts (~16 significant bits), V^T from ds_read_b64_tr_b16 transpose reads.
// At a piece's end the wave writes the normalised partial output and log2-sum-exp of its
// 32 rows to slot ((piece * subs + sub) * Hkv + head).
template <int D>
struct DecodeSmem {
  static constexpr int kVStride = D + 16;   // bf16 per V row: 32-byte pad, conflict-free tr reads
  static constexpr int kQStride = D + 8;    // bf16 per Q row: 16-byte pad
  uint16_t v[kWaves][kTile * kVStride];     // each wave's own slices
  uint16_t q[kWaves][32 * kQStride];
};

struct Pass {
  int kb, nv, bA, bB;
  bool in;
};

template <int D, bool IDX_LDS>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void gqa_decode_kernel(GqaDecodeArgs a) {
  constexpr int KS = D / 16;   // QK k-steps (32x32x16)
  constexpr int MT = D / 32;   // O^T tiles of 32 dims
  constexpr int DC = D / 8;    // 16-byte chunks per V row
  constexpr int VG = D / 64;   // (4 keys x 8 dims) V groups per lane per pass
  using Sm = DecodeSmem<D>;
  __shared__ __attribute__((aligned(16))) Sm sm;
  __shared__ int prog[kWaves];
  __shared__ int idx_s[kDecodeIdxLds];
  __shared__ int wsum_s[kWaves];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  if (lane == 0) prog[wave] = 0;
  int done = 0;
  const int c32 = lane & 31, h32 = lane >> 5;
  const int Hq = a.num_q_heads, Hkv = a.num_kv_heads;
  const int G = Hq / Hkv, T = a.q_per_seq, R = T * G;
  const int M = a.dims.members, NS = a.dims.subs;
  const int m = c32 / R, rr = c32 % R;
  const int t = rr / G, hh = rr % G;
  const size_t head_stride = (size_t)16 * D;
  uint16_t* vs = sm.v[wave];
  uint16_t* qs = sm.q[wave];
  const int NG = a.dims.n_groups, NC = a.dims.n_chunks, n_regions = NG * NC;
  // Region starts (n_regions + 1) and group piece starts (NG + 1): with IDX_LDS numbered
  // here, in LDS, by every workgroup alike from the plan's pass counts (workgroup 0 also
  // stores the piece starts for the combine); otherwise read from the workspace, where
  // decode_scan_kernel numbered them (too many regions for the LDS index).  The numbering
  // is the same either way.
  int* const rs_l = idx_s;
  int* const ps_l = idx_s + n_regions + 1;
  const int32_t* const rs = IDX_LDS ? rs_l : a.region_start;
  const int32_t* const ps = IDX_LDS ? ps_l : a.piece_start;
  if (IDX_LDS) {
    int running = 0;
    for (int base = 0; base < n_regions; base += kThreads) {
      const int r = base + tid;
      int total;
      const int off = block_exclusive_scan<kWaves>(r < n_regions ? a.n_passes[r] : 0, wsum_s, &total);
      if (r < n_regions) rs_l[r] = running + off;
      running += total;
    }
    if (tid == 0) rs_l[n_regions] = running;
    __syncthreads();                                // rs_l complete
    const long P0 = running, N0 = active_wgs(gridDim.x, P0);
    int pieces = 0;
    for (int base = 0; base < NG; base += kThreads) {
      const int g = base + tid;
      int cnt = 0;
      if (g < NG) {
        const int s0 = rs_l[g * NC], s1 = rs_l[(g + 1) * NC];
        cnt = s1 > s0 ? wg_of(s1 - 1, P0, N0) - wg_of(s0, P0, N0) + 1 : 0;
      }
      int total;
      const int off = block_exclusive_scan<kWaves>(cnt, wsum_s, &total);
      if (g < NG) ps_l[g] = pieces + off;
      pieces += total;
    }
    if (tid == 0) ps_l[NG] = pieces;
    __syncthreads();
    if (blockIdx.x == 0)
      for (int g = tid; g <= NG; g += kThreads) a.piece_start[g] = ps_l[g];
  }
  const long P = rs[n_regions];
  const long N = active_wgs(gridDim.x, P);
  const int w = blockIdx.x;
  if (w >= N) return;                               // fewer passes than workgroups
  const int lo = (int)wg_bound(w, P, N), hi = (int)wg_bound(w + 1, P, N);
  // this wave's (head, sub-range): NS = 8 / Hkv sub-ranges when Hkv divides 8, else one
  // and heads wave, wave + 8, ...
  const int sub = NS > 1 ? wave / Hkv : 0;
  const int h_first = NS > 1 ? wave % Hkv : wave;
  const int rlo = region_of(rs, n_regions, lo);
  const int m16 = lane & 15, gq = (lane >> 4) & 1;

  // The groups meeting [lo, hi), one piece each: passes px0 .. px1 - 1 of the compact
  // numbering (this wave's sub-range of the group's share), which may cross the group's
  // region boundaries.
  for (int grp = rlo / NC; grp < NG; ++grp) {
    const int gs = rs[grp * NC], ge = rs[(grp + 1) * NC];
    if (gs >= hi) break;
    const int x0 = max(gs, lo), x1 = min(ge, hi);
    if (x0 >= x1) continue;                         // a group with no pass
    const int piece = ps[grp] + (w - wg_of(gs, P, N));
    const int px0 = x0 + (int)((long)(x1 - x0) * sub / NS);
    const int px1 = x0 + (int)((long)(x1 - x0) * (sub + 1) / NS);
    // a region at or before the one holding px0 (rlo holds lo <= px0; a later group's
    // first pass is in its first region)
    const int rc0 = max(grp * NC, rlo);
    const int rc0_s = __builtin_amdgcn_readfirstlane(rs[rc0]);
    const int rc0_e = __builtin_amdgcn_readfirstlane(rs[rc0 + 1]);
    const int s = grp * M + m;
    const bool row_ok = (m < M) && (s < a.num_seqs);
    const int L = row_ok ? min(max(a.context_len[s], 0), a.max_context_len) : 0;
    const int pos = L - T + t;                      // keys <= pos are visible

    for (int g = h_first; g < Hkv; g += (NS > 1 ? Hkv : kWaves)) {
      const uint16_t* qrow = qs + c32 * Sm::kQStride + 8 * h32;
      f32x16 acc[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[mt][i] = 0.f;
      float m_run = -INFINITY, l_run = 0.f;

      // ---- passes px0 .. px1 - 1; the descriptor of the next pass to issue is loaded one
      // pass ahead.  Passes [rs0, rs1) of the numbering are region rc's, stored from
      // rc * region_cap; a pass past rs1 moves the cursor on (it stays inside the group:
      // every pass below px1 <= ge belongs to one of its regions).
      int it = px0, rc = rc0, rs0 = rc0_s, rs1 = rc0_e;
      auto pass_desc = [&]() -> u32x4 {
        while (rs1 <= it) {
          ++rc;
          rs0 = rs1;
          rs1 = __builtin_amdgcn_readfirstlane(rs[rc + 1]);
        }
        return ld16(a.passes + ((size_t)rc * a.dims.region_cap + (it - rs0)) * 4);
      };
      u32x4 dnext = it < px1 ? pass_desc() : u32x4{0, 0, 0, 0};
      auto next_pass = [&](Pass& Pp) -> bool {
        if (it >= px1) return false;
        const u32x4 d = dnext;
        ++it;
        if (it < px1) dnext = pass_desc();
        const uint32_t d0 = __builtin_amdgcn_readfirstlane(d.x);
        Pp.kb = (int)(d0 & ~31u);
        Pp.nv = (int)(d0 & 31u) + 1;
        Pp.bA = (int)__builtin_amdgcn_readfirstlane(d.y);
        Pp.bB = (int)__builtin_amdgcn_readfirstlane(d.z);
        const uint32_t mask = __builtin_amdgcn_readfirstlane(d.w);
        Pp.in = row_ok && ((mask >> m) & 1u);
        return true;
      };
      // K rows straight into the A operand (lane: key c32 of the pass); V as 4 keys x 8 dims.
      // Interior passes (both blocks present, all 32 keys hold data) take an unconditional path.
      auto issue = [&](const Pass& Pp, u32x4 (&kf)[KS], u32x4 (&vr)[VG][4]) {
        if (Pp.bA >= 0 && Pp.bB >= 0 && Pp.nv == kTile) {
          const int blk = c32 < 16 ? Pp.bA : Pp.bB;
          const uint16_t* kp = a.k + ((size_t)blk * Hkv + g) * head_stride + (size_t)(c32 & 15) * D + 8 * h32;
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) kf[ks] = ld16(kp + 16 * ks);
#pragma unroll
          for (int j = 0; j < VG; ++j) {
            const int gi = lane + 64 * j, dc = gi % DC, kg = gi / DC;
            const int vb = kg < 4 ? Pp.bA : Pp.bB;
            const uint16_t* vp = a.v + ((size_t)vb * Hkv + g) * head_stride + (size_t)(4 * (kg & 3)) * D + 8 * dc;
#pragma unroll
            for (int e = 0; e < 4; ++e) vr[j][e] = ld16(vp + (size_t)e * D);
          }
          return;
        }
        const int blk = c32 < 16 ? Pp.bA : Pp.bB;
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
          const int vb = kg < 4 ? Pp.bA : Pp.bB;
          if (vb >= 0) {
            const uint16_t* vp = a.v + ((size_t)vb * Hkv + g) * head_stride + (size_t)(4 * (kg & 3)) * D + 8 * dc;
#pragma unroll
            for (int e = 0; e < 4; ++e)
              vr[j][e] = (4 * kg + e < Pp.nv) ? ld16(vp + (size_t)e * D) : u32x4{0, 0, 0, 0};
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) vr[j][e] = u32x4{0, 0, 0, 0};
          }
        }
      };
      Pass nxt;
      u32x4 kfA[KS], kfB[KS], vr_n[VG][4];
      // One pass with its K in kf; the next pass is issued into kf_o (ping-pong) and vr_n.
      auto process = [&](u32x4 (&kf)[KS], u32x4 (&kf_o)[KS]) -> bool {
        const Pass cur = nxt;
        // The two waves of a SIMD share its issue slots and the older one wins ties, so
        // with equal work the younger one would finish long after (measured: a 92 us
        // spread of 380).  A wave behind its workgroup's average progress (its LDS
        // counter against everyone's; a stale read only delays the decision) takes the
        // higher issue priority until it has caught up.
        {
          ++done;
          if (lane == 0) prog[wave] = done;
          int sum = 0;
#pragma unroll
          for (int i = 0; i < kWaves; ++i) sum += prog[i];
          if (__builtin_amdgcn_readfirstlane(done * kWaves < sum)) __builtin_amdgcn_s_setprio(2);
          else __builtin_amdgcn_s_setprio(0);
        }
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
        // ---- S^T = K Q^T (Q^T fragments from the wave's LDS slice)
        f32x16 sacc = mfma32x32x16(kf[0], *reinterpret_cast<const u32x4*>(qrow), f32x16{});
#pragma unroll
        for (int ks = 1; ks < KS; ++ks)
          sacc = mfma32x32x16(kf[ks], *reinterpret_cast<const u32x4*>(qrow + 16 * ks), sacc);
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
        // the V slice written above is read back by this wave only
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          // P = P_hi + P_lo, both bf16: the pair carries ~16 significant bits of P
          u32x4 ph, pl;
#pragma unroll
          for (int wv = 0; wv < 4; ++wv) {
            const float a0 = sacc[8 * ks + 2 * wv], a1 = sacc[8 * ks + 2 * wv + 1];
            const uint32_t hv = pack_bf16x2(a0, a1);
            ph[wv] = hv;
            pl[wv] = pack_bf16x2(a0 - __uint_as_float(hv << 16), a1 - __uint_as_float(hv & 0xffff0000u));
          }
          // this lane's keys: kbase + 0..3 and kbase + 8..11 (the P^T register order)
          const int kbase = 16 * ks + 4 * h32;
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            const uint16_t* vp = vs + (kbase + (m16 >> 2)) * Sm::kVStride + 32 * mt + 16 * gq + 4 * (m16 & 3);
            const u32x2 lo2 = lds_read_tr16(vp);
            const u32x2 hi2 = lds_read_tr16(vp + 8 * Sm::kVStride);
            const u32x4 va = u32x4{lo2.x, lo2.y, hi2.x, hi2.y};
            acc[mt] = mfma32x32x16(va, ph, acc[mt]);
            acc[mt] = mfma32x32x16(va, pl, acc[mt]);
          }
        }
        // the LDS slice is rewritten by the next pass only after these reads
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        return more;
      };
      bool have = next_pass(nxt);
      if (have) issue(nxt, kfA, vr_n);
      // ---- this head's 32 query rows -> the wave's Q slice (read back as Q^T fragments,
      // B operand: lane = row c32); rows of members that do not exist are zero.  Loaded
      // after the first pass's K and V are on their way, so the two latencies overlap.
      for (int c = lane; c < 32 * DC; c += 64) {
        const int qr = c / DC, dc = c % DC;
        const int mr = qr / R, rr2 = qr % R, sr = grp * M + mr;
        u32x4 v = {0, 0, 0, 0};
        if (mr < M && sr < a.num_seqs)
          v = ld16(a.q + ((size_t)(sr * T + rr2 / G) * Hq + g * G + rr2 % G) * D + 8 * dc);
        st16(qs + qr * Sm::kQStride + 8 * dc, v);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      while (have) {
        have = process(kfA, kfB);
        if (!have) break;
        have = process(kfB, kfA);
      }

      // ---- the piece's partial: every row is written (rows of members that do not exist
      // get lse = -inf); the combine reads only the rows of real sequences
      const float l_tot = l_run + __shfl_xor(l_run, 32);
      const size_t pidx = (((size_t)piece * NS + sub) * Hkv + g) * 32 + c32;
      const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
      float* op = a.part_o + pidx * D;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          *reinterpret_cast<f32x4*>(op + 32 * mt + 8 * q4 + 4 * h32) =
              f32x4{acc[mt][4 * q4] * inv, acc[mt][4 * q4 + 1] * inv, acc[mt][4 * q4 + 2] * inv, acc[mt][4 * q4 + 3] * inv};
      if (h32 == 0) a.part_lse[pidx] = l_tot > 0.f ? m_run + __log2f(l_tot) : -INFINITY;
      // the Q slice is rewritten for the next head or piece only after this wave's reads
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }  // heads of this wave
  }  // regions
}

}  // namespace

int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

hipError_t launch_gqa_decode_plan(const GqaDecodeArgs& a, hipStream_t stream) {
  const unsigned regions = (unsigned)a.dims.n_groups * a.dims.n_chunks;
  if (regions == 0) return hipSuccess;
  hipLaunchKernelGGL(decode_plan_kernel, dim3(regions), dim3(256), 0, stream, a);
  if (!a.dims.scan_in_kernel) hipLaunchKernelGGL(decode_scan_kernel, dim3(1), dim3(1024), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_gqa_decode(const GqaDecodeArgs& a, hipStream_t stream) {
  if (a.dims.n_groups == 0 || a.dims.n_chunks == 0) return hipSuccess;
  const dim3 grid(a.dims.grid), block(kThreads);
  if (a.head_dim == 128) {
    if (a.dims.scan_in_kernel) hipLaunchKernelGGL((gqa_decode_kernel<128, true>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((gqa_decode_kernel<128, false>), grid, block, 0, stream, a);
  } else {
    if (a.dims.scan_in_kernel) hipLaunchKernelGGL((gqa_decode_kernel<64, true>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((gqa_decode_kernel<64, false>), grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------
// 4. Fixed-order combine of partials: for each (sequence, row) with n partials,
//   o = sum_j 2^(lse_j - M) o_j / sum_j 2^(lse_j - M),  M = max_j lse_j.
// A workgroup takes one (sequence, row): its threads form JL lanes over the partials
// (lane jl takes j = jl, jl + JL, ...) times D/4 lanes over the dimensions; each lane
// keeps an online (max, sum, weighted sum) and the JL lane states are merged in lane
// order, so the result is identical run to run.
namespace {
constexpr int kCombineBatch = 8;   // partials loaded per lane before they are used

__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  __shared__ f32x4 num_s[256];
  __shared__ float m_s[256], den_s[256];
  int row = blockIdx.x % a.rows, s = blockIdx.x / a.rows;
  const int D = a.head_dim, DV4 = D / 4, JL = 256 / DV4;
  const int tid = threadIdx.x, jl = tid / DV4, d4 = tid % DV4;
  size_t base;
  long stride;
  int n;
  if (a.pf_q_start != nullptr) {
    // split-K prefill: block (sequence, new token j, head); s becomes the packed token row
    const int seq = s / a.pf_max_new, j = s % a.pf_max_new;
    const int nl = min(a.pf_new_len[seq], a.pf_max_new);
    if (j >= nl) return;                           // no such token: nothing to write
    const int cached = a.pf_cached[seq];
    const int total = min(cached + nl, a.pf_max_total);
    const int vis = min(cached + j, total - 1) + 1;  // keys the token sees
    n = vis > 0 ? min((vis + a.split - 1) / a.split, a.max_splits) : 0;
    base = ((size_t)seq * a.pf_max_new + j) * a.max_splits * a.rows + row;   // token slot
    s = a.pf_q_start[seq] + j;                                                // output row
    stride = a.rows;
  } else if (a.piece_start != nullptr) {
    // GQA decode: the group's pieces are consecutive, each with `subs` sub-range partials,
    // in pass order; slot ((piece * subs + sub) * Hkv + head), row m * R + t * G + hq % G
    const int Hq = a.rows / a.q_per_seq, G = Hq / a.num_kv_heads, R = a.q_per_seq * G;
    const int t = row / Hq, hq = row % Hq, head = hq / G;
    const int g = s / a.members, m = s % a.members;
    const int u0 = a.piece_start[g], u1 = a.piece_start[g + 1];
    n = (u1 - u0) * a.subs;
    base = ((size_t)u0 * a.subs * a.num_kv_heads + head) * 32 + m * R + t * G + hq % G;
    stride = (long)a.num_kv_heads * 32;
  } else {
    const int L = min(max(a.context_len[s], 0), a.max_context_len);
    n = L > 0 ? (L + a.split - 1) / a.split : 0;
    base = (size_t)s * a.max_splits * a.rows + row;
    stride = a.rows;
  }
  float mx = -INFINITY, den = 0.f;
  f32x4 num = {0.f, 0.f, 0.f, 0.f};
  for (int j0 = jl; j0 < n; j0 += JL * kCombineBatch) {
    float lj[kCombineBatch];
    f32x4 oj[kCombineBatch];
#pragma unroll
    for (int b = 0; b < kCombineBatch; ++b) {
      const int j = j0 + b * JL;
      const size_t slot = base + (size_t)j * stride;
      lj[b] = j < n ? a.part_lse[slot] : -INFINITY;
      oj[b] = j < n ? *reinterpret_cast<const f32x4*>(a.part_o + slot * D + 4 * d4) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int b = 0; b < kCombineBatch; ++b) {
      if (lj[b] == -INFINITY) continue;
      if (lj[b] > mx) {
        const float sc = mx == -INFINITY ? 0.f : fast_exp2(mx - lj[b]);
        den *= sc;
        num *= sc;
        mx = lj[b];
      }
      const float w = fast_exp2(lj[b] - mx);
      den += w;
      num += w * oj[b];
    }
  }
  num_s[tid] = num;
  m_s[tid] = mx;
  den_s[tid] = den;
  __syncthreads();
  if (jl != 0) return;
  float M = -INFINITY;
  for (int k = 0; k < JL; ++k) M = fmaxf(M, m_s[k * DV4 + d4]);
  float tden = 0.f;
  f32x4 tnum = {0.f, 0.f, 0.f, 0.f};
  if (M != -INFINITY) {
    for (int k = 0; k < JL; ++k) {
      const float mk = m_s[k * DV4 + d4];
      if (mk == -INFINITY) continue;
      const float w = fast_exp2(mk - M);
      tden += w * den_s[k * DV4 + d4];
      tnum += w * num_s[k * DV4 + d4];
    }
  }
  const float inv = tden > 0.f ? 1.f / tden : 0.f;
  uint16_t* out = a.out + ((size_t)s * a.rows + row) * D + 4 * d4;
  const f32x2 lo = {tnum[0] * inv, tnum[1] * inv}, hi = {tnum[2] * inv, tnum[3] * inv};
  *reinterpret_cast<u32x2*>(out) = u32x2{pack_bf16x2(lo.x, lo.y), pack_bf16x2(hi.x, hi.y)};
  if (a.lse != nullptr && d4 == 0)
    a.lse[(size_t)s * a.rows + row] = tden > 0.f ? (M + __log2f(tden)) * kLn2 : -INFINITY;
}
}  // namespace

hipError_t launch_combine(const CombineArgs& a, hipStream_t stream) {
  const unsigned grid = (unsigned)a.num_seqs * (a.pf_q_start != nullptr ? (unsigned)a.pf_max_new : 1u) * a.rows;
  if (grid == 0) return hipSuccess;
  if (a.head_dim % 4 != 0 || a.head_dim / 4 > 256 || 256 % (a.head_dim / 4) != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(combine_kernel, dim3(grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pa
