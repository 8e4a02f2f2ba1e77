// Device-side helpers shared by the gfx950 kernels: vector types, MFMA wrappers, format
// conversions and the block-table walk.
//
// MFMA lane layouts used throughout (64-lane wavefront):
//   v_mfma_f32_16x16x32_bf16:  A[16 x 32]: lane l holds row l%16, k = 8*(l/16) .. +7
//                              B[32 x 16]: lane l holds col l%16, k = 8*(l/16) .. +7
//                              C[16 x 16]: lane l holds col l%16, rows 4*(l/16) + i, i<4
//   v_mfma_f32_32x32x16_bf16:  A[32 x 16]: lane l holds row l%32, k = 8*(l/32) .. +7
//                              B[16 x 32]: lane l holds col l%32, k = 8*(l/32) .. +7
//                              C[32 x 32]: lane l holds col l%32,
//                                          rows 8*(i/4) + 4*(l/32) + i%4, i<16
// The reduction index k may be relabelled freely as long as A and B agree, which the
// kernels use to feed softmax probabilities straight from a C tile into the next MFMA.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma32x32x16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// fp16 variants, used for P.V: probabilities in [0, 1] keep 11 significant bits in fp16
// (8 in bf16), and V converts to fp16 exactly (see below).
__device__ __forceinline__ f32x4 mfma16x16x32_f16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                 __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma32x32x16_f16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                 __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// Two floats -> packed fp16x2, round to nearest even (v_cvt_pk_f16_f32).
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
}

// Packed bf16x2 -> packed fp16x2.  Exact for |x| in [2^-14, 65504] (8 significant bits fit
// in 11); smaller magnitudes become fp16 subnormals (absolute error < 2^-25) and larger
// ones saturate to +-65504 (round toward zero never overflows to infinity).
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t u) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(__uint_as_float(u << 16),
                                                                  __uint_as_float(u & 0xffff0000u)));
}

// ---- bf16 operands on the FP8 MFMA.  A row of bf16 values is scaled by 2^qs, which brings
// its largest magnitude into [128, 256), and each scaled value x is split into two E4M3
// terms, hi = RN(x) and lo = RN(x - hi).  x has 8 significant bits and each term 4, and the
// residual x - hi is a multiple of x's last bf16 place, so hi + lo = x exactly when that
// place is at least E4M3's subnormal step 2^-9, i.e. for |x| >= 2^-2 (elements at least 2^-9
// of the row's largest); below that the absolute error is at most 2^-10 (scaled units).

// qs for a row whose largest |bf16| has the bit pattern amax (sign cleared): 7 - (its
// unbiased exponent), kept where 2^qs and 2^-qs are normal floats; 0 for an all-zero row.
__device__ __forceinline__ int split_scale_exp(uint32_t amax) {
  return amax == 0u ? 0 : min(126, max(-126, 134 - (int)(amax >> 7)));
}

// 2^e as a float, e in [-126, 127].
__device__ __forceinline__ float exp2i(int e) { return __uint_as_float((uint32_t)(127 + e) << 23); }

// Largest |bf16| bit pattern among the 8 values of a 16-byte word group.
__device__ __forceinline__ uint32_t bf16x8_absmax_bits(u32x4 v, uint32_t m) {
#pragma unroll
  for (int w = 0; w < 4; ++w) m = max(m, max(v[w] & 0x7fffu, (v[w] >> 16) & 0x7fffu));
  return m;
}

// Four bf16 values (two words, low half first) times up = 2^qs -> their E4M3 hi terms and
// lo terms, one word of four bytes each (byte i = value i).
__device__ __forceinline__ void bf16x4_split_e4m3(uint32_t v0, uint32_t v1, float up, uint32_t& hb, uint32_t& lb) {
  const float x0 = __uint_as_float(v0 << 16) * up, x1 = __uint_as_float(v0 & 0xffff0000u) * up;
  const float x2 = __uint_as_float(v1 << 16) * up, x3 = __uint_as_float(v1 & 0xffff0000u) * up;
  uint32_t h = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
  h = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, (int)h, true);
  const f32x2 h01 = __builtin_amdgcn_cvt_pk_f32_fp8((int)h, false);
  const f32x2 h23 = __builtin_amdgcn_cvt_pk_f32_fp8((int)h, true);
  uint32_t l = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(x0 - h01.x, x1 - h01.y, 0, false);
  l = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(x2 - h23.x, x3 - h23.y, (int)l, true);
  hb = h;
  lb = l;
}

typedef int i32x8 __attribute__((ext_vector_type(8)));

// Eight 16-byte-aligned words as one FP8 MFMA operand (32 bytes).
__device__ __forceinline__ i32x8 as_i32x8(u32x4 a, u32x4 b) {
  return i32x8{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
}

// FP8 (E4M3) MFMAs with fp32 accumulation: the two operands hold 32 bytes a lane in the same
// byte order (the reduction index is laid out alike for A and B, measured), so any order
// used for both pairs the right elements.  Zero scale operands select the unscaled
// instruction.
__device__ __forceinline__ f32x16 mfma32x32x64_fp8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16x16x128_fp8(i32x8 a, i32x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}
// A in E4M3 (32 bytes a lane, unscaled: code 127), B in E2M1 (16 bytes a lane in the first
// four words, element j in nibble j) with the lane's E8M0 code b_code scaling its 32
// elements.  The two operands' lane layouts differ (measured): B's lane group g holds
// reduction indices 32 g .. + 31, A's holds 16 g .. + 15 (bytes 0-15) and 64 + 16 g .. + 15
// (bytes 16-31).
__device__ __forceinline__ f32x4 mfma16x16x128_fp8_fp4(i32x8 a, i32x8 b, int b_code, f32x4 c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 4, 0, 127, 0, b_code);
}

// Four OCP E4M3FN bytes -> four fp16, exact (every E4M3 value is an fp16 normal).  The
// gfx950 scaled converter with scale 1 writes two fp16 per instruction.
#ifndef PA_CVT_SCALED
#define PA_CVT_SCALED 1
#endif
__device__ __forceinline__ u32x2 fp8x4_to_f16x4(uint32_t src) {
  u32x2 r;
#if PA_CVT_SCALED
  r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)src, 1.0f, false));
  r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)src, 1.0f, true));
#else
  const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)src, false);
  const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)src, true);
  r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo.x, lo.y));
  r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(hi.x, hi.y));
#endif
  return r;
}

// Two floats -> packed bf16x2 (round to nearest even).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// Four OCP E4M3FN bytes -> four bf16 (exact: every E4M3 value is a bf16 value), two per
// instruction with the gfx950 scaled converter (scale 1); otherwise the fp32 converter
// and the upper halves.
__device__ __forceinline__ u32x2 fp8x4_to_bf16x4(uint32_t src) {
  u32x2 r;
#if PA_CVT_SCALED
  r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)src, 1.0f, false));
  r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)src, 1.0f, true));
#else
  f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)src, false);
  f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)src, true);
  r.x = __builtin_amdgcn_perm(__float_as_uint(lo.y), __float_as_uint(lo.x), 0x07060302u);
  r.y = __builtin_amdgcn_perm(__float_as_uint(hi.y), __float_as_uint(hi.x), 0x07060302u);
#endif
  return r;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ds_read_b64_tr_b16 (LDS transpose read, 16-bit elements).  Within each group of 16
// lanes, lane n receives element n%4 of the 8-byte reads of lanes 4j + n/4 (j = 0..3).  So
// when lane m of a group reads 4 consecutive elements at row r0 + m/4, column c0 + 4*(m%4)
// of a row-major LDS matrix, lane n gets column c0 + n of rows r0 .. r0+3: a 4 x 16 block
// arrives transposed, one column per lane -- the MFMA operand layout with the reduction
// index (rows) in the lane's registers.
__device__ __forceinline__ u32x2 lds_read_tr16(const uint16_t* p) {
  typedef short i16x4 __attribute__((ext_vector_type(4)));
  auto* lp = (__attribute__((address_space(3))) i16x4*)((__attribute__((address_space(3))) uint16_t*)p);
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(lp));
}

// Unaligned-free 16-byte global load / store helpers.
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// Physical block of logical block `lb` of a sequence, or -1 when lb is past the
// sequence's blocks or the table entry is out of range (the caller then uses zeros).
__device__ __forceinline__ int32_t phys_block(const int32_t* __restrict__ bt_row, int32_t lb,
                                              int32_t n_lblocks, int32_t num_blocks) {
  if (lb >= n_lblocks) return -1;
  int32_t b = bt_row[lb];
  return (b >= 0 && b < num_blocks) ? b : -1;
}

// Workgroups are dispatched round-robin over the 8 XCDs (each with its own L2).  This
// maps the hardware id so that consecutive logical ids run on the same XCD, which keeps
// workgroups that read the same KV range together in one L2.
__device__ __forceinline__ int32_t xcd_swizzle(int32_t hw_id, int32_t n) {
  const int32_t n8 = n & ~7;
  if (hw_id >= n8) return hw_id;
  return (hw_id & 7) * (n8 >> 3) + (hw_id >> 3);
}

// Work units of per_unit consecutive logical ids, dealt to the 8 XCDs round robin: XCD x
// runs units x, x + 8, x + 16, ... (all ids of a unit on one XCD, sharing its L2), so the
// XCDs get statistically equal work even when units differ in size along the id order.
// Bijective on [0, n); ids past the last whole round of 8 units map to themselves.
__device__ __forceinline__ int32_t xcd_unit_swizzle(int32_t hw_id, int32_t n, int32_t per_unit) {
  const int32_t n8 = (n / (8 * per_unit)) * (8 * per_unit);
  if (hw_id >= n8) return hw_id;
  const int32_t k = hw_id >> 3;
  return ((k / per_unit) * 8 + (hw_id & 7)) * per_unit + k % per_unit;
}

// LDS-DMA of 16 (or 4) bytes per lane: lane l's global bytes land at LDS byte address
// lds_dst + 16 l (4 l); lds_dst must be the same for every lane.  Issued as inline assembly, so the compiler
// does not track these LDS writes: it would otherwise wait for every outstanding DMA
// before any LDS read it cannot prove disjoint (the S exchange and the transpose reads
// among them), draining the pipeline.  The pipeline waits explicitly (wait_vm0, then a
// barrier) before any wave reads what a DMA wrote.  M0 holds the LDS base; nothing else
// in these kernels uses M0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void* src, uint32_t lds_dst) {
  const uint32_t l = __builtin_amdgcn_readfirstlane(lds_dst);
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(l) : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void* src, uint32_t lds_dst) {
  const uint32_t l = __builtin_amdgcn_readfirstlane(lds_dst);
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(src), "s"(l) : "memory", "m0");
}
// LDS byte address of a pointer into a __shared__ object.
__device__ __forceinline__ uint32_t lds_u32(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
#pragma clang diagnostic pop
// Wait until no vector-memory operation of this wave is outstanding (gfx9 s_waitcnt
// encoding: vmcnt 0, expcnt and lgkmcnt left at their maxima).
// (also a compiler barrier: no LDS read of DMA data moves above it)
__device__ __forceinline__ void wait_vm0() {
  __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));
  asm volatile("" ::: "memory");
}
// Workgroup barrier that orders LDS accesses only.  A full __syncthreads() also waits for
// outstanding vector-memory operations -- here the LDS-DMA of a later tile, still in
// flight on purpose.
// (An LDS-scoped fence is no help: LDS-DMA writes count as LDS writes, so it waits for
// them too.)  The compiler-level memory clobbers keep LDS accesses on their side of it.
__device__ __forceinline__ void barrier_lds() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt and expcnt left at their maxima
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ float wave_max_xor(float v, int lanes) {
  for (int o = lanes >> 1; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ float wave_sum_xor(float v, int lanes) {
  for (int o = lanes >> 1; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

}  // namespace pa
