// Per-query top-k over indexer scores: radix select on order-preserving 32-bit keys,
// then an index-ordered compaction.
//
// Sources: GLM-5.3 report (aisoku.org), "What's new" and "How to try" (2,048 tokens per
// query token); vLLM AgentX article (news.ainew.jp), "Closing the loop: kernels" (top-k
// is a known hotspot).  The selection is exact: the k largest scores, ties broken toward
// the lower token index, returned in ascending token order.
//
// One workgroup (8 waves) per query row.  Four passes build 256-bin histograms of one
// 8-bit digit (most significant first) among the scores that match the digits found so
// far, in per-wave LDS sub-histograms; each pass fixes one digit of T, the key of the
// k-th largest score, and how many of the elements equal to T must be taken.  A last
// pass walks the row in index order, 512 scores at a time, and writes every index with
// key > T plus the first (k - #greater) indices with key == T, using two block-wide
// prefix sums per chunk.  -0.0 is keyed as +0.0, so the two zeros tie as equal values.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;

__device__ __forceinline__ uint32_t score_key(float f) {
  const uint32_t u = __float_as_uint(f + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
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

__global__ __launch_bounds__(kThreads) void topk_kernel(TopkArgs a) {
  __shared__ uint32_t hist[kWaves][256];
  __shared__ uint32_t sh_prefix, sh_kk;
  __shared__ int wsum[kWaves];
  const int tid = threadIdx.x, wave = tid >> 6;
  const int row = blockIdx.x;
  const int valid = max(0, min(a.valid_len[row], a.max_valid));
  const int k = a.k;
  int32_t* out = a.out + (size_t)row * k;
  const float* sc = a.scores + (size_t)row * a.row_stride;
  if (valid <= k) {
    for (int j = tid; j < k; j += kThreads) out[j] = j < valid ? j : -1;
    return;
  }
  uint32_t prefix = 0, mask = 0, kk = (uint32_t)k;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int j = tid; j < kWaves * 256; j += kThreads) (&hist[0][0])[j] = 0u;
    __syncthreads();
    for (int t = tid; t < valid; t += kThreads) {
      const uint32_t u = score_key(sc[t]);
      if ((u & mask) == prefix) atomicAdd(&hist[wave][(u >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid < 256) {
      uint32_t c = 0;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) c += hist[w][tid];
      hist[0][tid] = c;
    }
    __syncthreads();
    if (tid == 0) {
      uint32_t acc = 0;
      int d = 255;
      for (; d > 0; --d) {
        if (acc + hist[0][d] >= kk) break;
        acc += hist[0][d];
      }
      sh_prefix = prefix | ((uint32_t)d << shift);
      sh_kk = kk - acc;
    }
    __syncthreads();
    prefix = sh_prefix;
    kk = sh_kk;
    mask |= 0xFFu << shift;
  }
  // prefix == T; kk elements equal to T are taken, lowest indices first.
  const uint32_t T = prefix;
  int eq_seen = 0, written = 0;
  for (int c0 = 0; c0 < valid; c0 += kThreads) {
    const int t = c0 + tid;
    uint32_t u = 0;
    if (t < valid) u = score_key(sc[t]);
    const int is_gt = (t < valid && u > T) ? 1 : 0;
    const int is_eq = (t < valid && u == T) ? 1 : 0;
    int eq_tot, take_tot;
    const int eq_rank = eq_seen + block_excl_scan(is_eq, wsum, eq_tot);
    const int take = is_gt | (is_eq & (eq_rank < (int)kk ? 1 : 0));
    const int slot = written + block_excl_scan(take, wsum, take_tot);
    if (take && slot < k) out[slot] = t;
    eq_seen += eq_tot;
    written += take_tot;
  }
}

}  // namespace

hipError_t launch_topk(const TopkArgs& a, hipStream_t stream) {
  if (a.n_rows == 0) return hipSuccess;
  hipLaunchKernelGGL(topk_kernel, dim3(a.n_rows), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pa
