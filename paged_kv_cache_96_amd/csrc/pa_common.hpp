// Device helpers shared by the paged-attention kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kLn2 = 0.69314718055994530942f;

// ---------------------------------------------------------------- bfloat16
// bf16 is carried as raw 16-bit patterns; widening to fp32 is exact.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two fp32 -> packed bf16 pair (lo, hi) with the hardware converter
// (v_cvt_pk_bf16_f32, round to nearest even).
__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
  f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// a.lo*b.lo + a.hi*b.hi + c with bf16 pairs (products exact, fp32 sum).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// ----------------------------------------------------------- streaming loads
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// 16-byte load with the non-temporal hint: data read exactly once (paged
// decode K/V) bypasses normal cache allocation, which on MI355X lifts the
// sustained HBM read rate well above that of ordinary loads.
__device__ __forceinline__ u32x4_t load_stream(const void *p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
}

// Word 3 of a raw (stride 0) buffer resource on gfx9-family GPUs: 32-bit
// data format, no swizzle.
constexpr int kBufferRsrcWord3 = 0x00020000;

// 16-byte non-temporal raw buffer load at byte offset `off`; offsets at or
// past the resource's num_records return zeros without a memory access.
__device__ __forceinline__ u32x4_t load_stream_buf(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, /*nt*/ 2);
}

// ------------------------------------------------------------ exponentials
// Scores are kept in base-2 units (scale already multiplied by log2 e), so
// every exponential is one hardware exp2.  exp2(-inf) = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// --------------------------------------------------------------- cross-lane
// DPP control words (gfx9 encoding).
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i of an 8-lane half row <- lane 7-i
constexpr int kDppMirror = 0x140;     // lane i of a 16-lane row <- lane 15-i
constexpr int kDppRor8 = 0x128;       // lane i of a 16-lane row <- lane (i+8)%16

// Values of the lane pair {l, l ^ 16} (permlane16 swap) and {l, l ^ 32}
// (permlane32 swap), lower lane first in every lane of the pair; VALU only,
// no LDS crossbar.
__device__ __forceinline__ void pair16(float x, float &lo, float &hi) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  lo = __uint_as_float(r[0]);
  hi = __uint_as_float(r[1]);
}
__device__ __forceinline__ void pair32(float x, float &lo, float &hi) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  lo = __uint_as_float(r[0]);
  hi = __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum16(float x) { float a, b; pair16(x, a, b); return a + b; }
__device__ __forceinline__ float sum32(float x) { float a, b; pair32(x, a, b); return a + b; }
__device__ __forceinline__ float max16(float x) { float a, b; pair16(x, a, b); return fmaxf(a, b); }
__device__ __forceinline__ float max32(float x) { float a, b; pair32(x, a, b); return fmaxf(a, b); }

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of N consecutive lanes; every lane of a group ends
// with the same value (float addition is commutative, and each step adds the
// same pair in both lanes).
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(N == 1 || N == 2 || N == 4 || N == 8 || N == 16 || N == 32 || N == 64, "N");
  if constexpr (N >= 2) x += dpp<kDppXor1>(x);
  if constexpr (N >= 4) x += dpp<kDppXor2>(x);
  if constexpr (N >= 8) x += dpp<kDppHalfMirror>(x);
  if constexpr (N >= 16) x += dpp<kDppMirror>(x);
  if constexpr (N >= 32) x = sum16(x);
  if constexpr (N >= 64) x = sum32(x);
  return x;
}

// Max over aligned groups of N consecutive lanes (every lane gets it).
template <int N>
__device__ __forceinline__ float group_max(float x) {
  static_assert(N == 1 || N == 2 || N == 4 || N == 8 || N == 16 || N == 32 || N == 64, "N");
  if constexpr (N >= 2) x = fmaxf(x, dpp<kDppXor1>(x));
  if constexpr (N >= 4) x = fmaxf(x, dpp<kDppXor2>(x));
  if constexpr (N >= 8) x = fmaxf(x, dpp<kDppHalfMirror>(x));
  if constexpr (N >= 16) x = fmaxf(x, dpp<kDppMirror>(x));
  if constexpr (N >= 32) x = max16(x);
  if constexpr (N >= 64) x = max32(x);
  return x;
}

// Reduce across lanes that differ only in bits >= log2(STRIDE) of the lane
// id (lanes l, l ^ STRIDE, l ^ 2*STRIDE, ...): combines the per-token-group
// partial states of one wave.
template <int STRIDE>
__device__ __forceinline__ float stride_sum(float x) {
  if constexpr (STRIDE <= 8) x += dpp<kDppRor8>(x);
  if constexpr (STRIDE <= 16) x = sum16(x);
  if constexpr (STRIDE <= 32) x = sum32(x);
  return x;
}
template <int STRIDE>
__device__ __forceinline__ float stride_max(float x) {
  if constexpr (STRIDE <= 8) x = fmaxf(x, dpp<kDppRor8>(x));
  if constexpr (STRIDE <= 16) x = max16(x);
  if constexpr (STRIDE <= 32) x = max32(x);
  return x;
}

}  // namespace pa
