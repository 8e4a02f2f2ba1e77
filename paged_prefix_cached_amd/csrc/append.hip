// Paged KV append: the new tokens of a step are written into their sequences' blocks,
// bf16 rows copied as they are, FP8 rows quantised per token.
//
// Sources: vLLM AgentX article (news.ainew.jp), "Hybrid KV cache management" -- one
// shared block pool, logical token t of a sequence in row t % block_size of physical
// block block_table[t / block_size], so an append is a scatter through the table.
// GLM-5.3 on 16xH200 report (aisoku.org), "Configuration and numbers" table (FP8 KV) and
// "What's new" (one latent KV row per token) -- the cache holds FP8.  The pages give no
// quantiser; the one here is per token: scale = amax / 448 (1 when the row is all zero),
// code = E4M3 round-to-nearest-even of x / scale in IEEE float32, clamped to +-448.
// The packed per-block layout ("Hybrid KV cache management", Figure 5) keeps the index
// keys as MXFP4 (the FP4 indexer): see append_mxfp4_kernel.
//
// Both kernels are grids of (token range, sequence); a sequence's rows are q_start[s] ..
// q_start[s] + new_len[s] - 1 of the packed input and go to logical positions
// cached_len[s] ... .  The work is pure HBM streaming: each input byte is read once and
// each pool byte written once, in 16-byte (bf16) or 8-byte (FP8) vector accesses.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kGqaTokensPerBlock = 8;
constexpr int kFp8WavesPerBlock = 4;   // one token per wave

// Where the new tokens of sequence s go.  The three per-sequence values are loaded
// together; then slot(j) needs one block-table load.
struct SeqAppend {
  int nl, q0, c0;
};

__device__ __forceinline__ SeqAppend seq_append(const AppendArgs& a, int s) {
  const int nl = a.new_len[s], q0 = a.q_start[s], c0 = a.cached_len[s];
  return {min(nl, a.max_new_len), q0, c0};
}

// Pool row (block * BS + row) of new token j, given the block id b of its logical block
// (read by the caller), or -1 when it has none (beyond new_len, an input row outside
// [0, n_tokens), a position outside the block table, or an out-of-range block id).
// *row_out gets the input row, 0 when there is none (row 0 exists: n_tokens >= 1), so
// that a load from it is always in bounds.
template <int BS>
__device__ __forceinline__ long dest_slot(const AppendArgs& a, const SeqAppend& q, int j, int b,
                                          int* row_out) {
  const int row = q.q0 + j;
  const int pos = q.c0 + j;
  const int lb = pos >> __builtin_ctz(BS);           // floor division
  const bool ok = (j < q.nl) & (row >= 0) & (row < a.n_tokens) & (pos >= 0) & (lb < a.bt_stride) &
                  (b >= 0) & (b < a.num_blocks);
  *row_out = ok ? row : 0;
  return ok ? (long)b * BS + (pos & (BS - 1)) : -1;
}

// Block-table entry lb of sequence s, clamped into the row so that the load is always in
// bounds (a clamped entry is never used: dest_slot rejects lb outside [0, bt_stride)).
__device__ __forceinline__ int bt_entry(const AppendArgs& a, int s, int lb) {
  return a.bt[(size_t)s * a.bt_stride + min(max(lb, 0), a.bt_stride - 1)];
}

// bf16 GQA pool [NB][Hkv][16][d]: a workgroup appends kGqaTokensPerBlock tokens of one
// sequence; thread r copies 16-byte chunk r of each token's K|V (2 * Hkv * d / 8 chunks).
// The destinations are resolved once, before any store, so the metadata loads are scalar;
// then every thread issues its loads for all the tokens before its first store (the
// compiler may not move a load past a store to the pool, which could alias the input).
__global__ __launch_bounds__(256) void append_gqa_kernel(AppendArgs a) {
  const int s = blockIdx.y;
  const int chunks = a.head_dim / 8;                 // 16-byte chunks per head row
  const int per_tok = a.num_kv_heads * chunks;       // chunks of one token's K (or V)
  const int j0 = blockIdx.x * kGqaTokensPerBlock;
  static_assert(kGqaTokensPerBlock <= 16, "a workgroup's tokens span at most two 16-token blocks");
  const SeqAppend sq = seq_append(a, s);
  const int lb0 = (sq.c0 + j0) >> 4;
  const int b0 = bt_entry(a, s, lb0), b1 = bt_entry(a, s, lb0 + 1);
  long slot[kGqaTokensPerBlock];
  int row[kGqaTokensPerBlock];
#pragma unroll
  for (int t = 0; t < kGqaTokensPerBlock; ++t)
    slot[t] = dest_slot<16>(a, sq, j0 + t, ((sq.c0 + j0 + t) >> 4) == lb0 ? b0 : b1, &row[t]);
  for (int r = threadIdx.x; r < 2 * per_tok; r += blockDim.x) {
    const int kv = r >= per_tok;
    const int hc = r - kv * per_tok;                 // head * chunks + chunk
    const int h = hc / chunks, c = hc - h * chunks;
    const uint16_t* src = (kv ? a.v_new : a.k_new) + 8 * hc;
    uint16_t* dst = (kv ? a.v_out : a.k_out) + (size_t)h * 16 * a.head_dim + 8 * c;
    u32x4 v[kGqaTokensPerBlock];
#pragma unroll
    for (int t = 0; t < kGqaTokensPerBlock; ++t) v[t] = ld16(src + (size_t)row[t] * per_tok * 8);
#pragma unroll
    for (int t = 0; t < kGqaTokensPerBlock; ++t) {
      if (slot[t] < 0) continue;
      const long blk = slot[t] >> 4, rr = slot[t] & 15;
      st16(dst + ((size_t)blk * a.num_kv_heads * 16 + rr) * a.head_dim, v[t]);
    }
  }
}

// FP8 pool [NB][64][D] + scales [NB][64]: one wave per token.  Lane l holds the 8-element
// chunks l, l + 64, ... of the row in registers (D <= 1024), so the row is read once.
template <int D>
__global__ __launch_bounds__(64 * kFp8WavesPerBlock) void append_fp8_kernel(AppendArgs a) {
  constexpr int kChunks = D / 8;
  constexpr int kPer = (kChunks + 63) / 64;
  const int s = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int j = blockIdx.x * kFp8WavesPerBlock + (threadIdx.x >> 6);
  const SeqAppend sq = seq_append(a, s);
  int row;
  const long slot = dest_slot<64>(a, sq, j, bt_entry(a, s, (sq.c0 + j) >> 6), &row);
  if (slot < 0) return;                              // the whole wave agrees
  const uint16_t* src = a.k_new + (size_t)row * D;
  float x[kPer][8];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int c = lane + 64 * i;
    u32x4 v = {0, 0, 0, 0};
    if (c < kChunks) v = ld16(src + 8 * c);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[i][2 * e] = __uint_as_float(w[e] << 16);
      x[i][2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
      amax = fmaxf(amax, fmaxf(fabsf(x[i][2 * e]), fabsf(x[i][2 * e + 1])));
    }
  }
  amax = wave_max_xor(amax, 64);
  // IEEE float32 division (correctly rounded): the code of every element is decided on
  // exactly the value x / scale.
  const float scale = amax > 0.f ? amax / 448.f : 1.f;
  const long blk = slot >> 6, r = slot & 63;
  uint8_t* dst = a.fp8_out + blk * a.blk_bytes + r * D;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int c = lane + 64 * i;
    if (c >= kChunks) continue;
    uint32_t packed[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float y[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) y[e] = fminf(fmaxf(x[i][4 * h + e] / scale, -448.f), 448.f);
      int p = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
      p = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], p, true);
      packed[h] = (uint32_t)p;
    }
    u32x2 o;
    o.x = packed[0];
    o.y = packed[1];
    *reinterpret_cast<u32x2*>(dst + 8 * c) = o;
  }
  if (lane == 0) *reinterpret_cast<float*>(a.scale_out + blk * a.sblk_bytes + 4 * r) = scale;
}

// MXFP4 rows (the index keys of the packed per-block layout), D = 128: one wave per token,
// lane l holds elements 2l and 2l + 1, so a group of 32 elements is 16 lanes.  Per group
// (OCP MX conversion): E8M0 code e = floor(log2 amax) - 2 + 127 -- the exponent field of
// amax minus 2 -- kept in [2, 252], 127 for an all-zero group; every element is scaled by
// 2^(127 - e) (exact) and rounded to the nearest E2M1 value, ties to the even code, with
// saturation at 6: the magnitude code is the number of rounding boundaries below |y|
// (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5; a tie at a boundary goes to the even side).
// Element 2j goes to the low nibble of byte j; the four scale codes follow the row.
__global__ __launch_bounds__(64 * kFp8WavesPerBlock) void append_mxfp4_kernel(AppendArgs a) {
  constexpr int D = 128;
  const int s = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int j = blockIdx.x * kFp8WavesPerBlock + (threadIdx.x >> 6);
  const SeqAppend sq = seq_append(a, s);
  int row;
  const long slot = dest_slot<64>(a, sq, j, bt_entry(a, s, (sq.c0 + j) >> 6), &row);
  if (slot < 0) return;                              // the whole wave agrees
  const uint32_t w = *reinterpret_cast<const uint32_t*>(a.k_new + (size_t)row * D + 2 * lane);
  const float x0 = __uint_as_float(w << 16), x1 = __uint_as_float(w & 0xffff0000u);
  float amax = fmaxf(fabsf(x0), fabsf(x1));
  amax = wave_max_xor(amax, 16);                     // the lane's group of 16 lanes
  const int field = (int)(__float_as_uint(amax) >> 23);
  const uint32_t e = amax > 0.f ? (uint32_t)min(max(field - 2, 2), 252) : 127u;
  const float inv = __uint_as_float((254u - e) << 23);   // 2^(127 - e)
  auto code = [&](float x) -> uint32_t {
    const float y = x * inv;
    const float m = fabsf(y);
    const uint32_t c = (uint32_t)(m > 0.25f) + (uint32_t)(m >= 0.75f) + (uint32_t)(m > 1.25f) +
                       (uint32_t)(m >= 1.75f) + (uint32_t)(m > 2.5f) + (uint32_t)(m >= 3.5f) +
                       (uint32_t)(m > 5.0f);
    return c | ((__float_as_uint(y) >> 28) & 8u);     // the sign bit
  };
  const uint32_t byte = code(x0) | (code(x1) << 4);
  // four lanes' bytes -> one 32-bit store
  const uint32_t b1 = __shfl_down(byte, 1), b2 = __shfl_down(byte, 2), b3 = __shfl_down(byte, 3);
  const long blk = slot >> 6, r = slot & 63;
  uint8_t* dst = a.fp8_out + blk * a.blk_bytes + r * (D / 2);
  if ((lane & 3) == 0)
    *reinterpret_cast<uint32_t*>(dst + lane) = byte | (b1 << 8) | (b2 << 16) | (b3 << 24);
  const uint32_t e1 = __shfl(e, 16), e2 = __shfl(e, 32), e3 = __shfl(e, 48);
  if (lane == 0)
    *reinterpret_cast<uint32_t*>(a.scale_out + blk * a.sblk_bytes + 4 * r) = e | (e1 << 8) | (e2 << 16) | (e3 << 24);
}

}  // namespace

hipError_t launch_append(const AppendArgs& a, hipStream_t stream) {
  if (a.num_seqs == 0 || a.max_new_len == 0) return hipSuccess;
  if (!a.is_fp8) {
    const dim3 grid((a.max_new_len + kGqaTokensPerBlock - 1) / kGqaTokensPerBlock, a.num_seqs);
    hipLaunchKernelGGL(append_gqa_kernel, grid, dim3(256), 0, stream, a);
    return hipGetLastError();
  }
  const dim3 grid((a.max_new_len + kFp8WavesPerBlock - 1) / kFp8WavesPerBlock, a.num_seqs);
  const dim3 block(64 * kFp8WavesPerBlock);
  if (a.mxfp4) {
    if (a.head_dim != 128) return hipErrorInvalidValue;
    hipLaunchKernelGGL(append_mxfp4_kernel, grid, block, 0, stream, a);
  } else if (a.head_dim == 576)
    hipLaunchKernelGGL(append_fp8_kernel<576>, grid, block, 0, stream, a);
  else if (a.head_dim == 128)
    hipLaunchKernelGGL(append_fp8_kernel<128>, grid, block, 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pa
