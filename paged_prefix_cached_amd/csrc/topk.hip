// Per-query top-k over indexer scores: the k largest scores of a row, ties broken toward
// the lower token index, returned in ascending token order (-1 padding when the row has
// fewer than k valid tokens).
//
// Sources: GLM-5.3 report (aisoku.org), "What's new" and "How to try" (2,048 tokens per
// query token); vLLM AgentX article (news.ainew.jp), "Closing the loop: kernels" (top-k
// is a known hotspot).
//
// Scores are compared through order-preserving 32-bit keys (-0.0 keyed as +0.0, so the
// two zeros tie).  One workgroup of 1,024 threads per row; the row is read twice:
//   1. a 4,096-bin LDS histogram of the top 12 key bits locates the bin b holding the
//      k-th largest key, with G keys above it;
//   2. in index order, keys above b set their bit in an LDS selection bitmap and keys in
//      b are appended, in index order, to an LDS candidate list;
// then, in LDS only: a radix select over the candidates' low 20 bits finds T, the k-th
// largest key, and how many keys equal to T to take; candidates above T and the first
// such ties (in index order) join the bitmap; a prefix sum over bitmap popcounts writes
// the selected indices in ascending order.
// Rows longer than the bitmap or whose bin b overflows the candidate list fall back to
// four 8-bit radix passes over the row plus an index-ordered compaction pass.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kBins = 4096;                 // top 12 key bits
constexpr int kMaxBits = 1 << 18;           // bitmap capacity (tokens per row)
constexpr int kWords = kMaxBits / 32;
constexpr int kCand = 3072;                 // candidate list capacity
static_assert(kBins <= 4 * kThreads, "bin search covers 4 bins a thread");

__device__ __forceinline__ uint32_t score_key(float f) {
  const uint32_t u = __float_as_uint(f + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// 16 consecutive scores from sc[e0 ..] as keys; positions at or past `valid` get flag 0.
// VEC: sc + e0 is 16-byte aligned (four 16-byte loads), else scalar loads.
template <bool VEC>
__device__ __forceinline__ void load16(const float* sc, int e0, int valid, float (&f)[16]) {
  if (VEC && e0 + 16 <= valid) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(sc + e0 + 4 * q);
      f[4 * q] = v.x; f[4 * q + 1] = v.y; f[4 * q + 2] = v.z; f[4 * q + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < 16; ++j) f[j] = e0 + j < valid ? sc[e0 + j] : 0.f;
  }
}

// Exclusive prefix sum over the workgroup; returns the exclusive value, sets total.
__device__ __forceinline__ int block_excl_scan(int v, int* wsum, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  int before = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const int sw = wsum[w];
    before += (w < wave) ? sw : 0;
    total += sw;
  }
  __syncthreads();
  return before + x - v;
}

struct TopkSmem {
  uint32_t hist[kBins];
  uint32_t bits[kWords];
  int32_t cidx[kCand];
  uint32_t ckey[kCand];
  int wsum[kWaves];
  uint32_t sh_bin, sh_kk, sh_n;
};

// Bin d of sm.hist[0..nbins) (nbins a multiple of 4, at most 4 * kThreads) with G keys in
// the bins above it and G < kk <= G + hist[d]: d -> sm.sh_bin, kk - G -> sm.sh_kk,
// hist[d] -> sm.sh_n.  Each thread sums a group of 4 bins; a block scan in reversed
// group order gives the count above every group.
__device__ void find_bin_from_top(TopkSmem& sm, int nbins, uint32_t kk) {
  const int g = nbins / 4 - 1 - (int)threadIdx.x;
  uint32_t c[4] = {0u, 0u, 0u, 0u};
  if (g >= 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) c[i] = sm.hist[4 * g + i];
  }
  int tot;
  int above = block_excl_scan((int)(c[0] + c[1] + c[2] + c[3]), sm.wsum, tot);
#pragma unroll
  for (int i = 3; i >= 0; --i) {
    if (g >= 0 && above < (int)kk && above + (int)c[i] >= (int)kk) {
      sm.sh_bin = (uint32_t)(4 * g + i);
      sm.sh_kk = kk - (uint32_t)above;
      sm.sh_n = c[i];
    }
    above += (int)c[i];
  }
  __syncthreads();
}

// Radix select on a prefix-filtered set held in the candidate list: the kk-th largest key
// among ckey[0..n) (all sharing the top 12 bits), as T and the number of keys equal to T
// that are taken.  Two passes over bits 19..8 (12 bits) and 7..0 (8 bits).
__device__ void select_in_candidates(TopkSmem& sm, int n, uint32_t kk, uint32_t& T, uint32_t& kk_eq) {
  const int tid = threadIdx.x;
  uint32_t prefix = sm.ckey[0] & 0xFFF00000u, mask = 0xFFF00000u;
  const int shifts[2] = {8, 0};
  const int widths[2] = {12, 8};
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int sh = shifts[pass], nb = 1 << widths[pass];
    for (int j = tid; j < nb; j += kThreads) sm.hist[j] = 0u;
    __syncthreads();
    for (int i = tid; i < n; i += kThreads) {
      const uint32_t u = sm.ckey[i];
      if ((u & mask) == prefix) atomicAdd(&sm.hist[(u >> sh) & (nb - 1)], 1u);
    }
    __syncthreads();
    find_bin_from_top(sm, nb, kk);
    prefix |= sm.sh_bin << sh;
    kk = sm.sh_kk;
    mask |= (uint32_t)(nb - 1) << sh;
    __syncthreads();
  }
  T = prefix;
  kk_eq = kk;
}

// Fallback: four 8-bit radix passes over the row, then an index-ordered compaction.
__device__ void topk_radix_row(TopkSmem& sm, const float* sc, int valid, int k, int32_t* out) {
  const int tid = threadIdx.x;
  uint32_t prefix = 0, mask = 0, kk = (uint32_t)k;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int j = tid; j < 256; j += kThreads) sm.hist[j] = 0u;
    __syncthreads();
    for (int t = tid; t < valid; t += kThreads) {
      const uint32_t u = score_key(sc[t]);
      if ((u & mask) == prefix) atomicAdd(&sm.hist[(u >> shift) & 255u], 1u);
    }
    __syncthreads();
    find_bin_from_top(sm, 256, kk);
    prefix |= sm.sh_bin << shift;
    kk = sm.sh_kk;
    mask |= 0xFFu << shift;
    __syncthreads();
  }
  const uint32_t T = prefix;
  int eq_seen = 0, written = 0;
  for (int c0 = 0; c0 < valid; c0 += kThreads) {
    const int t = c0 + tid;
    uint32_t u = 0;
    if (t < valid) u = score_key(sc[t]);
    const int is_gt = (t < valid && u > T) ? 1 : 0;
    const int is_eq = (t < valid && u == T) ? 1 : 0;
    int eq_tot, take_tot;
    const int eq_rank = eq_seen + block_excl_scan(is_eq, sm.wsum, eq_tot);
    const int take = is_gt | (is_eq & (eq_rank < (int)kk ? 1 : 0));
    const int slot = written + block_excl_scan(take, sm.wsum, take_tot);
    if (take && slot < k) out[slot] = t;
    eq_seen += eq_tot;
    written += take_tot;
  }
}

__global__ __launch_bounds__(kThreads) void topk_kernel(TopkArgs a) {
  __shared__ TopkSmem sm;
  const int tid = threadIdx.x, lane = tid & 63;
  const int row = blockIdx.x;
  const int valid = max(0, min(a.valid_len[row], a.max_valid));
  const int k = a.k;
  int32_t* out = a.out + (size_t)row * k;
  const float* sc = a.scores + (size_t)row * a.row_stride;
  if (valid <= k) {
    for (int j = tid; j < k; j += kThreads) out[j] = j < valid ? j : -1;
    return;
  }
  if (valid > kMaxBits) {
    topk_radix_row(sm, sc, valid, k, out);
    return;
  }

  // Both passes walk the row in super-chunks of 16 consecutive scores per thread
  // (16,384 per workgroup step), the next super-chunk's loads in flight while the current
  // one is processed.
  constexpr int kPer = 16, kSuper = kThreads * kPer;
  const bool vec = ((reinterpret_cast<uintptr_t>(sc) & 15u) == 0);
  const int n_super = (valid + kSuper - 1) / kSuper;

  // ---- pass 1: histogram of the top 12 key bits
  for (int j = tid; j < kBins; j += kThreads) sm.hist[j] = 0u;
  __syncthreads();
  {
    float cur[kPer], nxt[kPer];
    if (vec) load16<true>(sc, kPer * tid, valid, cur); else load16<false>(sc, kPer * tid, valid, cur);
    for (int sI = 0; sI < n_super; ++sI) {
      const int e0 = sI * kSuper + kPer * tid;
      if (sI + 1 < n_super) {
        if (vec) load16<true>(sc, e0 + kSuper, valid, nxt); else load16<false>(sc, e0 + kSuper, valid, nxt);
      }
#pragma unroll
      for (int j = 0; j < kPer; ++j)
        if (e0 + j < valid) atomicAdd(&sm.hist[score_key(cur[j]) >> 20], 1u);
#pragma unroll
      for (int j = 0; j < kPer; ++j) cur[j] = nxt[j];
    }
  }
  __syncthreads();
  // bin b with G keys above it and G < k <= G + hist[b]
  find_bin_from_top(sm, kBins, (uint32_t)k);
  const uint32_t b = sm.sh_bin, kk = sm.sh_kk;
  const int nb = (int)sm.sh_n;
  if (nb > kCand) {
    __syncthreads();
    topk_radix_row(sm, sc, valid, k, out);
    return;
  }

  // ---- pass 2: bitmap of keys above b, index-ordered candidate list of keys in b
  const int nwords = (valid + 31) / 32;
  for (int j = tid; j < nwords; j += kThreads) sm.bits[j] = 0u;
  __syncthreads();
  int n_cand = 0;
  {
    float cur[kPer], nxt[kPer];
    if (vec) load16<true>(sc, kPer * tid, valid, cur); else load16<false>(sc, kPer * tid, valid, cur);
    for (int sI = 0; sI < n_super; ++sI) {
      const int e0 = sI * kSuper + kPer * tid;
      if (sI + 1 < n_super) {
        if (vec) load16<true>(sc, e0 + kSuper, valid, nxt); else load16<false>(sc, e0 + kSuper, valid, nxt);
      }
      uint32_t above_bits = 0u;
      int ncand = 0;
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const uint32_t hb = score_key(cur[j]) >> 20;
        const bool in = e0 + j < valid;
        above_bits |= (in && hb > b) ? (1u << j) : 0u;
        ncand += (in && hb == b) ? 1 : 0;
      }
      // two threads' 16 bits form one bitmap word (elements e0 .. e0 + 31)
      const uint32_t other = __shfl_xor(above_bits, 1);
      if ((lane & 1) == 0 && (e0 >> 5) < nwords) sm.bits[e0 >> 5] = above_bits | (other << 16);
      int tot;
      int pos = n_cand + block_excl_scan(ncand, sm.wsum, tot);
      if (ncand) {
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
          const uint32_t u = score_key(cur[j]);
          if (e0 + j < valid && (u >> 20) == b) {
            sm.cidx[pos] = e0 + j;
            sm.ckey[pos] = u;
            ++pos;
          }
        }
      }
      n_cand += tot;
#pragma unroll
      for (int j = 0; j < kPer; ++j) cur[j] = nxt[j];
    }
  }
  __syncthreads();

  // ---- resolve T among the candidates; add the chosen ones to the bitmap
  uint32_t T, kk_eq;
  select_in_candidates(sm, n_cand, kk, T, kk_eq);
  {
    int tie_seen = 0;
    for (int i0 = 0; i0 < n_cand; i0 += kThreads) {
      const int i = i0 + tid;
      const uint32_t u = i < n_cand ? sm.ckey[i] : 0u;
      const bool gt = i < n_cand && u > T;
      const bool eq = i < n_cand && u == T;
      int tot;
      const int rank = tie_seen + block_excl_scan(eq ? 1 : 0, sm.wsum, tot);
      if (gt || (eq && rank < (int)kk_eq)) {
        const int t = sm.cidx[i];
        atomicOr(&sm.bits[t >> 5], 1u << (t & 31));
      }
      tie_seen += tot;
    }
  }
  __syncthreads();

  // ---- compaction: each thread owns a run of consecutive bitmap words
  {
    const int per = (nwords + kThreads - 1) / kThreads;
    const int w_begin = min(nwords, tid * per), w_end = min(nwords, w_begin + per);
    int cnt = 0;
    for (int w = w_begin; w < w_end; ++w) cnt += __popc(sm.bits[w]);
    int tot;
    int slot = block_excl_scan(cnt, sm.wsum, tot);
    for (int w = w_begin; w < w_end; ++w) {
      uint32_t x = sm.bits[w];
      while (x != 0u) {
        const int bit = __ffs(x) - 1;
        x &= x - 1u;
        if (slot < k) out[slot] = 32 * w + bit;
        ++slot;
      }
    }
  }
}

}  // namespace

hipError_t launch_topk(const TopkArgs& a, hipStream_t stream) {
  if (a.n_rows == 0) return hipSuccess;
  hipLaunchKernelGGL(topk_kernel, dim3(a.n_rows), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pa
