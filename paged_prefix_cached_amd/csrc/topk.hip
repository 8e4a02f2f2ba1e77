// Per-query top-k over indexer scores: the k largest scores of a row, ties broken toward
// the lower token index, returned in ascending token order (-1 padding when the row has
// fewer than k valid tokens).
//
// Sources: GLM-5.3 report (aisoku.org), "What's new" and "How to try" (2,048 tokens per
// query token); vLLM AgentX article (news.ainew.jp), "Closing the loop: kernels" (top-k
// is a known hotspot).
//
// Scores are compared through order-preserving 32-bit keys (-0.0 keyed as +0.0, so the
// two zeros tie).  One workgroup of 1,024 threads per row.
//
// One read (rows of at least kOneReadMin tokens, k <= kCand / 4): a sample of 4,096
// scores from 16 evenly spaced runs of the row gives, by a two-level LDS histogram, a key
// threshold tau that about 2k of the row's keys reach.  The row is then read once; every
// key >= tau is appended (key, token) to an LDS candidate list, each wave reserving its
// slots with one LDS atomic per 16,384-score step, so the pass has no barrier.  If at
// least k and at most kCand keys reached tau, the list holds the whole top k (the k-th
// largest key of the row is >= tau); a radix select over the list finds T, the k-th
// largest key, and how many keys equal to T to take; the taken ties (lowest tokens first,
// through an index-ordered scan of an LDS bitmap) and the keys above T set their bits in
// the bitmap, and a prefix sum over its popcounts writes the tokens in ascending order.
// Otherwise (the sample misled: too few or too many keys reached tau) the row takes the
// two-read path below.
//
// Two reads (shorter rows, and the fallback):
//   1. a 4,096-bin LDS histogram of the top 12 key bits locates the bin b holding the
//      k-th largest key, with G keys above it;
//   2. in index order, keys above b set their bit in the bitmap and keys in b are
//      appended, in index order, to the candidate list;
// then, in LDS only: a radix select over the candidates' low 20 bits finds T and the
// number of ties to take; candidates above T and the first such ties (in index order)
// join the bitmap, which is compacted as above.
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
constexpr int kCand = 8192;                 // candidate list capacity
constexpr int kSampleRun = 256;             // sample: one run of 256 scores per wave (4 a lane)
constexpr int kSample = kWaves * kSampleRun;  // 4,096 sampled scores
constexpr int kOneReadMin = 32768;          // shortest row that tries the one-read path
constexpr int kMinRank = 64;                // smallest sample rank used for the threshold
constexpr int kPer = 16;                    // scores per thread and step
constexpr int kSuper = kThreads * kPer;     // scores per workgroup step
static_assert(kBins <= 4 * kThreads, "bin search covers 4 bins a thread");
static_assert(kOneReadMin / kWaves >= kSampleRun, "sample runs do not overlap");

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

__device__ __forceinline__ void load16v(bool vec, const float* sc, int e0, int valid, float (&f)[16]) {
  if (vec) load16<true>(sc, e0, valid, f); else load16<false>(sc, e0, valid, f);
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
  int n_cand;
};

// Bin d of sm.hist[0..nbins) (nbins a multiple of 4, at most 4 * kThreads) with G keys in
// the bins above it and G < kk <= G + hist[d]: d -> sm.sh_bin, kk - G -> sm.sh_kk,
// hist[d] -> sm.sh_n.  Each thread sums a group of 4 bins; a block scan in reversed
// group order gives the count above every group.  The caller guarantees kk <= the total.
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

// Radix select in LDS: the kk-th largest key among ckey[0..n) whose bits under `mask` equal
// `prefix`, over the key fields from `first` on (bits 31..20, 19..8, 7..0).  Returns T,
// the number of keys equal to T that are taken (kk_eq) and the number of keys equal to T
// among the filtered ones (n_eq).
__device__ void select_kth(TopkSmem& sm, int n, uint32_t kk, int first, uint32_t prefix, uint32_t mask,
                           uint32_t& T, uint32_t& kk_eq, uint32_t& n_eq) {
  const int tid = threadIdx.x;
  const int shifts[3] = {20, 8, 0};
  const int widths[3] = {12, 12, 8};
  uint32_t cnt = 0;
  for (int pass = first; pass < 3; ++pass) {
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
    cnt = sm.sh_n;
    mask |= (uint32_t)(nb - 1) << sh;
    __syncthreads();
  }
  T = prefix;
  kk_eq = kk;
  n_eq = cnt;
}

// The bitmap's set bits, in ascending token order, to out[0..k): each thread owns a run
// of consecutive words.
__device__ void write_bitmap(TopkSmem& sm, int nwords, int k, int32_t* out) {
  const int tid = threadIdx.x;
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

// One read of the row (see the file comment).  Returns false, uniformly over the
// workgroup and with nothing written to out, when the sampled threshold did not leave
// between k and kCand candidates; the caller then runs the two-read path.
// Requires kOneReadMin <= valid <= kMaxBits and k <= kCand / 4.
__device__ bool topk_one_read(TopkSmem& sm, const float* sc, int valid, int k, int32_t* out, bool vec) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n_super = (valid + kSuper - 1) / kSuper;
  // The first step's loads go out before the sample is processed.
  float cur[kPer], nxt[kPer];
  load16v(vec, sc, kPer * tid, valid, cur);

  // ---- sample: run w (wave w) starts at w (valid - 256) / 15, rounded down to 4 scores
  const int r0 = (int)(((long long)wave * (valid - kSampleRun) / (kWaves - 1)) & ~3ll);
  uint32_t skey[4];
  if (vec) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(sc + r0 + 4 * lane);
    skey[0] = score_key(v.x); skey[1] = score_key(v.y); skey[2] = score_key(v.z); skey[3] = score_key(v.w);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) skey[i] = score_key(sc[r0 + 4 * lane + i]);
  }
  for (int j = tid; j < kBins; j += kThreads) sm.hist[j] = 0u;
  if (tid == 0) sm.n_cand = 0;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) atomicAdd(&sm.hist[skey[i] >> 20], 1u);
  __syncthreads();
  // rank in the sample whose key about 2k of the row's keys reach (at least kMinRank, so
  // that the count stays close to its expectation)
  const int want = (int)(((long long)2 * k * kSample + valid - 1) / valid);
  const uint32_t rank = (uint32_t)min(kSample, max(kMinRank, want));
  find_bin_from_top(sm, kBins, rank);
  const uint32_t b12 = sm.sh_bin, rr = sm.sh_kk;
  for (int j = tid; j < 256; j += kThreads) sm.hist[j] = 0u;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if ((skey[i] >> 20) == b12) atomicAdd(&sm.hist[(skey[i] >> 12) & 255u], 1u);
  __syncthreads();
  find_bin_from_top(sm, 256, rr);
  const uint32_t tau = (b12 << 20) | (sm.sh_bin << 12);

  // ---- the row, once: keys >= tau to the candidate list (slots reserved per wave)
  for (int sI = 0; sI < n_super; ++sI) {
    const int e0 = sI * kSuper + kPer * tid;
    if (sI + 1 < n_super) load16v(vec, sc, e0 + kSuper, valid, nxt);
    uint32_t accm = 0u;                                // bit j: score j reaches tau
    int tot = 0;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const bool acc = e0 + j < valid && score_key(cur[j]) >= tau;
      accm |= acc ? (1u << j) : 0u;
      tot += __popcll(__ballot(acc));
    }
    if (tot > 0) {                                     // wave-uniform
      int base = 0;
      if (lane == 0) base = atomicAdd(&sm.n_cand, tot);
      int slot = __shfl(base, 0);
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const bool acc = (accm >> j) & 1u;
        const uint64_t bal = __ballot(acc);
        if (acc) {
          const int s_j = slot + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                                 __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
          if (s_j < kCand) {
            sm.ckey[s_j] = score_key(cur[j]);
            sm.cidx[s_j] = e0 + j;
          }
        }
        slot += __popcll(bal);
      }
    }
#pragma unroll
    for (int j = 0; j < kPer; ++j) cur[j] = nxt[j];
  }
  __syncthreads();
  const int n = sm.n_cand;
  if (n < k || n > kCand) return false;

  // ---- T, the k-th largest key among the candidates, and the ties to take
  uint32_t T, kk_eq, n_eq;
  select_kth(sm, n, (uint32_t)k, 0, 0u, 0u, T, kk_eq, n_eq);
  const int nwords = (valid + 31) / 32;
  for (int j = tid; j < nwords; j += kThreads) sm.bits[j] = 0u;
  __syncthreads();
  if (n_eq != kk_eq) {
    // more keys equal T than are taken: keep the kk_eq lowest tokens among them
    for (int i = tid; i < n; i += kThreads)
      if (sm.ckey[i] == T) atomicOr(&sm.bits[sm.cidx[i] >> 5], 1u << (sm.cidx[i] & 31));
    __syncthreads();
    const int per = (nwords + kThreads - 1) / kThreads;
    const int w_begin = min(nwords, tid * per), w_end = min(nwords, w_begin + per);
    int cnt = 0;
    for (int w = w_begin; w < w_end; ++w) cnt += __popc(sm.bits[w]);
    int tot;
    int rank_t = block_excl_scan(cnt, sm.wsum, tot);
    for (int w = w_begin; w < w_end; ++w) {
      uint32_t x = sm.bits[w], keep = 0u;
      while (x != 0u) {
        const uint32_t low = x & (0u - x);
        x ^= low;
        if (rank_t < (int)kk_eq) keep |= low;
        ++rank_t;
      }
      sm.bits[w] = keep;
    }
    __syncthreads();
    for (int i = tid; i < n; i += kThreads)
      if (sm.ckey[i] > T) atomicOr(&sm.bits[sm.cidx[i] >> 5], 1u << (sm.cidx[i] & 31));
  } else {
    for (int i = tid; i < n; i += kThreads)
      if (sm.ckey[i] >= T) atomicOr(&sm.bits[sm.cidx[i] >> 5], 1u << (sm.cidx[i] & 31));
  }
  __syncthreads();
  write_bitmap(sm, nwords, k, out);
  return true;
}

// Two reads of the row (see the file comment).  Requires k < valid <= kMaxBits.
__device__ void topk_two_reads(TopkSmem& sm, const float* sc, int valid, int k, int32_t* out, bool vec) {
  const int tid = threadIdx.x, lane = tid & 63;
  // Both passes walk the row in steps of 16 consecutive scores per thread (16,384 per
  // workgroup step), the next step's loads in flight while the current one is processed.
  const int n_super = (valid + kSuper - 1) / kSuper;

  // ---- pass 1: histogram of the top 12 key bits
  for (int j = tid; j < kBins; j += kThreads) sm.hist[j] = 0u;
  __syncthreads();
  {
    float cur[kPer], nxt[kPer];
    load16v(vec, sc, kPer * tid, valid, cur);
    for (int sI = 0; sI < n_super; ++sI) {
      const int e0 = sI * kSuper + kPer * tid;
      if (sI + 1 < n_super) load16v(vec, sc, e0 + kSuper, valid, nxt);
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
    load16v(vec, sc, kPer * tid, valid, cur);
    for (int sI = 0; sI < n_super; ++sI) {
      const int e0 = sI * kSuper + kPer * tid;
      if (sI + 1 < n_super) load16v(vec, sc, e0 + kSuper, valid, nxt);
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

  // ---- resolve T among the candidates (all in bin b); add the chosen ones to the bitmap
  uint32_t T, kk_eq, n_eq;
  select_kth(sm, n_cand, kk, 1, b << 20, 0xFFF00000u, T, kk_eq, n_eq);
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
  write_bitmap(sm, nwords, k, out);
}

__global__ __launch_bounds__(kThreads) void topk_kernel(TopkArgs a) {
  __shared__ TopkSmem sm;
  const int tid = threadIdx.x;
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
  const bool vec = ((reinterpret_cast<uintptr_t>(sc) & 15u) == 0);
  if (valid >= kOneReadMin && k <= kCand / 4) {
    if (topk_one_read(sm, sc, valid, k, out, vec)) return;
    __syncthreads();
  }
  topk_two_reads(sm, sc, valid, k, out, vec);
}

}  // namespace

hipError_t launch_topk(const TopkArgs& a, hipStream_t stream) {
  if (a.n_rows == 0) return hipSuccess;
  hipLaunchKernelGGL(topk_kernel, dim3(a.n_rows), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pa
