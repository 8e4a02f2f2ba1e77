// Per-query top-k over indexer scores: the k largest scores of a row, ties broken toward
// the lower token index, returned in ascending token order (-1 padding when the row has
// fewer than k valid tokens).
//
// Sources: GLM-5.3 report (aisoku.org), "What's new" and "How to try" (2,048 tokens per
// query token); vLLM AgentX article (news.ainew.jp), "Closing the loop: kernels" (top-k
// is a known hotspot).
//
// Scores are compared through order-preserving 32-bit keys (-0.0 keyed as +0.0, so the
// two zeros tie).  One workgroup of 512 threads per row, two workgroups per CU (72 KB of
// LDS each), so one row's selection runs while the other row is being read.
//
// A row is selected through a key threshold tau that at least k of its keys reach:
//   1. tau: rows of at least kOneReadMin tokens with k <= kCand / 4 take it from a sample of
//      4,096 scores (8 evenly spaced runs of 512) by a two-level LDS histogram (top 11 key
//      bits, then the next 9 inside the chosen bin), aimed at about 2k keys; other rows take
//      the bin of the k-th largest key from a full-row 2,048-bin histogram (one more read);
//   2. one pass over the row appends every key >= tau (key, token) to an LDS candidate list,
//      each wave reserving its slots with one LDS atomic per 8,192-score step (no barrier);
//   3. if at least k and at most kCand keys reached tau, the list holds the whole top k (the
//      k-th largest key is >= tau): a three-pass radix select (11 + 11 + 10 bits) over the
//      list finds T, the k-th largest key, and how many keys equal to T to take; each
//      candidate's class (above T, equal, below) is folded into its token entry, and the
//      keys' LDS is then reused as a token bitmap: the taken ties (lowest tokens first,
//      through an index-ordered popcount scan) and the keys above T set their bits, and a
//      prefix sum over the popcounts writes the tokens in ascending order.
// A sampled tau that leaves fewer than k or more than kCand candidates falls back to the
// full-histogram tau; a bin holding more than kCand keys above the threshold, or a row
// longer than the bitmap, falls back to four 8-bit radix passes over the row plus an
// index-ordered compaction pass.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kThreads = 512;               // two workgroups per CU
constexpr int kWaves = kThreads / 64;
constexpr int kBins = 2048;                 // top 11 key bits
constexpr int kMaxBits = 1 << 18;           // bitmap capacity (tokens per row)
constexpr int kWords = kMaxBits / 32;
constexpr int kCand = 8192;                 // candidate list capacity
constexpr int kSampleRun = 512;             // sample: one run of 512 scores per wave (8 a lane)
constexpr int kSample = kWaves * kSampleRun;  // 4,096 sampled scores
constexpr int kOneReadMin = 32768;          // shortest row that tries the sampled threshold
constexpr int kMinRank = 64;                // smallest sample rank used for the threshold
constexpr int kPer = 16;                    // scores per thread and step
constexpr int kSuper = kThreads * kPer;     // scores per workgroup step
constexpr uint32_t kTokMask = (1u << 30) - 1;  // token bits of a candidate entry
static_assert(kBins <= 4 * kThreads, "bin search covers 4 bins a thread");
static_assert(kWords == kCand, "the bitmap reuses the candidates' key array");
static_assert(kOneReadMin / kWaves >= kSampleRun, "sample runs do not overlap");

__device__ __forceinline__ uint32_t score_key(float f) {
  const uint32_t u = __float_as_uint(f + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// 16 consecutive scores from sc[e0 ..]; positions at or past `valid` read as 0.
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
  uint32_t cidx[kCand];                     // candidate tokens (bits 30-31: class after the select)
  union {
    uint32_t ckey[kCand];                   // candidate keys, until T is known
    uint32_t bits[kWords];                  // then the token bitmap
  };
  int wsum[kWaves];
  uint32_t sh_bin, sh_kk, sh_n;
  int n_cand;
};

// Bin d of hist[0..nbins) (sm.hist unless given; nbins a multiple of 4, at most 4 * kThreads) with G keys in
// the bins above it and G < kk <= G + hist[d]: d -> sm.sh_bin, kk - G -> sm.sh_kk,
// hist[d] -> sm.sh_n.  Each thread sums a group of 4 bins; a block scan in reversed
// group order gives the count above every group.  The caller guarantees kk <= the total.
__device__ void find_bin_from_top(TopkSmem& sm, int nbins, uint32_t kk, const uint32_t* hist = nullptr) {
  if (hist == nullptr) hist = sm.hist;
  const int g = nbins / 4 - 1 - (int)threadIdx.x;
  uint32_t c[4] = {0u, 0u, 0u, 0u};
  if (g >= 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) c[i] = hist[4 * g + i];
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
    find_bin_from_top(sm, 256, kk);           // its last barrier follows every histogram read
    prefix |= sm.sh_bin << shift;
    kk = sm.sh_kk;
    mask |= 0xFFu << shift;
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

// tau from a sample of the row (see the file comment); the first step's loads are issued
// by the caller before this runs.  Requires kOneReadMin <= valid.
__device__ uint32_t sampled_tau(TopkSmem& sm, const float* sc, int valid, int k, bool vec) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // run w (wave w) starts at w (valid - 512) / 7, rounded down to 4 scores; lane l takes
  // scores 4 l .. + 3 and 256 + 4 l .. + 3 of it
  const int r0 = (int)(((long long)wave * (valid - kSampleRun) / (kWaves - 1)) & ~3ll);
  uint32_t skey[8];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const int e = r0 + 256 * hh + 4 * lane;
    if (vec) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(sc + e);
      skey[4 * hh] = score_key(v.x); skey[4 * hh + 1] = score_key(v.y);
      skey[4 * hh + 2] = score_key(v.z); skey[4 * hh + 3] = score_key(v.w);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) skey[4 * hh + i] = score_key(sc[e + i]);
    }
  }
  // first level in sm.hist, second level in the (still unused) candidate array; both and the
  // candidate count are cleared under one barrier
  uint32_t* hist2 = sm.cidx;
  for (int j = tid; j < kBins; j += kThreads) sm.hist[j] = 0u;
  for (int j = tid; j < 512; j += kThreads) hist2[j] = 0u;
  if (tid == 0) sm.n_cand = 0;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 8; ++i) atomicAdd(&sm.hist[skey[i] >> 21], 1u);
  __syncthreads();
  // rank in the sample whose key about 2k of the row's keys reach (at least kMinRank, so
  // that the count stays close to its expectation)
  const int want = (int)(((long long)2 * k * kSample + valid - 1) / valid);
  const uint32_t rank = (uint32_t)min(kSample, max(kMinRank, want));
  find_bin_from_top(sm, kBins, rank);
  const uint32_t b11 = sm.sh_bin, rr = sm.sh_kk;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    if ((skey[i] >> 21) == b11) atomicAdd(&hist2[(skey[i] >> 12) & 511u], 1u);
  __syncthreads();
  find_bin_from_top(sm, 512, rr, hist2);
  return (b11 << 21) | (sm.sh_bin << 12);
}

// tau = the lowest key of the bin holding the k-th largest key (a full-row histogram of
// the top 11 key bits; one read of the row).  Returns false when the keys from that bin
// up number more than kCand.  Requires k < valid.
__device__ bool exact_tau(TopkSmem& sm, const float* sc, int valid, int k, bool vec, uint32_t& tau) {
  const int tid = threadIdx.x;
  const int n_super = (valid + kSuper - 1) / kSuper;
  for (int j = tid; j < kBins; j += kThreads) sm.hist[j] = 0u;
  if (tid == 0) sm.n_cand = 0;
  __syncthreads();
  float cur[kPer], nxt[kPer];
  load16v(vec, sc, kPer * tid, valid, cur);
  for (int sI = 0; sI < n_super; ++sI) {
    const int e0 = sI * kSuper + kPer * tid;
    if (sI + 1 < n_super) load16v(vec, sc, e0 + kSuper, valid, nxt);
#pragma unroll
    for (int j = 0; j < kPer; ++j)
      if (e0 + j < valid) atomicAdd(&sm.hist[score_key(cur[j]) >> 21], 1u);
#pragma unroll
    for (int j = 0; j < kPer; ++j) cur[j] = nxt[j];
  }
  __syncthreads();
  find_bin_from_top(sm, kBins, (uint32_t)k);
  // keys from the bin up: the (k - kk) above it plus the bin's own
  const int above_and_bin = k - (int)sm.sh_kk + (int)sm.sh_n;
  tau = sm.sh_bin << 21;
  return above_and_bin <= kCand;
}

// Steps 2 and 3 of the file comment for a threshold tau (sampled_tau or exact_tau, which
// also clear sm.n_cand).  cur holds the first step's scores (loads issued by the caller).  Returns false, uniformly over the workgroup and with
// nothing written to out, when fewer than k or more than kCand keys reached tau.
__device__ bool select_from(TopkSmem& sm, const float* sc, int valid, int k, int32_t* out, bool vec, uint32_t tau,
                            float (&cur)[kPer]) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int n_super = (valid + kSuper - 1) / kSuper;
  float nxt[kPer];                                     // sm.n_cand was cleared with tau's histogram
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
            sm.cidx[s_j] = (uint32_t)(e0 + j);
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

  // ---- T, the k-th largest key among the candidates (radix select, LDS histograms over
  // bits 31..21, 20..10, 9..0), and the ties to take
  uint32_t prefix = 0u, mask = 0u, kk = (uint32_t)k, n_eq = 0u;
  {
    const int shifts[3] = {21, 10, 0};
    const int widths[3] = {11, 11, 10};
    for (int pass = 0; pass < 3; ++pass) {
      const int sh = shifts[pass], nb = 1 << widths[pass];
      for (int j = tid; j < nb; j += kThreads) sm.hist[j] = 0u;
      __syncthreads();
      for (int i = tid; i < n; i += kThreads) {
        const uint32_t u = sm.ckey[i];
        if ((u & mask) == prefix) atomicAdd(&sm.hist[(u >> sh) & (nb - 1)], 1u);
      }
      __syncthreads();
      // find_bin_from_top ends with a barrier after every histogram read, and the next pass
      // rewrites sm.sh_* only after further barriers, so no barrier is needed here
      find_bin_from_top(sm, nb, kk);
      prefix |= sm.sh_bin << sh;
      kk = sm.sh_kk;
      n_eq = sm.sh_n;
      mask |= (uint32_t)(nb - 1) << sh;
    }
  }
  const uint32_t T = prefix, kk_eq = kk;
  // each candidate's class into its token entry: 2 above T, 1 equal, 0 below
  for (int i = tid; i < n; i += kThreads) {
    const uint32_t u = sm.ckey[i];
    sm.cidx[i] |= (u > T ? 2u : (u == T ? 1u : 0u)) << 30;
  }
  __syncthreads();
  // the keys are no longer needed: their array becomes the bitmap
  const int nwords = (valid + 31) / 32;
  for (int j = tid; j < nwords; j += kThreads) sm.bits[j] = 0u;
  __syncthreads();
  if (n_eq != kk_eq) {
    // more keys equal T than are taken: keep the kk_eq lowest tokens among them
    for (int i = tid; i < n; i += kThreads) {
      const uint32_t e = sm.cidx[i];
      if ((e >> 30) == 1u) atomicOr(&sm.bits[(e & kTokMask) >> 5], 1u << (e & 31));
    }
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
    for (int i = tid; i < n; i += kThreads) {
      const uint32_t e = sm.cidx[i];
      if ((e >> 30) == 2u) atomicOr(&sm.bits[(e & kTokMask) >> 5], 1u << (e & 31));
    }
  } else {
    for (int i = tid; i < n; i += kThreads) {
      const uint32_t e = sm.cidx[i];
      if ((e >> 30) != 0u) atomicOr(&sm.bits[(e & kTokMask) >> 5], 1u << (e & 31));
    }
  }
  __syncthreads();
  // ---- the bitmap's set bits, in ascending token order, to out[0..k): each thread owns a
  // run of consecutive words
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
  return true;
}

__global__ __launch_bounds__(kThreads, 4) void topk_kernel(TopkArgs a) {
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
  float cur[kPer];
  if (valid >= kOneReadMin && k <= kCand / 4) {
    load16v(vec, sc, kPer * tid, valid, cur);          // in flight while the sample is processed
    const uint32_t tau = sampled_tau(sm, sc, valid, k, vec);
    if (select_from(sm, sc, valid, k, out, vec, tau, cur)) return;
    __syncthreads();
  }
  uint32_t tau;
  if (exact_tau(sm, sc, valid, k, vec, tau)) {
    __syncthreads();
    load16v(vec, sc, kPer * tid, valid, cur);
    if (select_from(sm, sc, valid, k, out, vec, tau, cur)) return;   // always: n >= k, n <= kCand
  }
  __syncthreads();
  topk_radix_row(sm, sc, valid, k, out);
}

}  // namespace

hipError_t launch_topk(const TopkArgs& a, hipStream_t stream) {
  if (a.n_rows == 0) return hipSuccess;
  hipLaunchKernelGGL(topk_kernel, dim3(a.n_rows), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pa
