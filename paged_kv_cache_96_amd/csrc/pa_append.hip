// K/V write path: every new token's key and value rows go to their physical
// slots in the page pool ("Reading vLLM's PagedAttention Kernel", section
// 3.2: the write side scatters tokens to flat slots page * page_size +
// offset, the read side gathers them back through the block table).
//
// One thread moves 16 bytes: a row of head_dim elements (128, 256 or 512
// bytes) is LANES consecutive threads, so a wave copies 1 KiB of source rows
// per instruction and each row lands as one contiguous run of its page.
// The slot of a token is read by the LANES threads of each of its rows (one
// cached load).  Tokens with a negative or out-of-pool slot are skipped.
// HBM bound: every byte is read once and written once.
//
// fp8 pages: each thread reads 8 bf16 elements and writes their 8 E4M3
// codes (8 bytes), so a row lands as LANES * 8 contiguous bytes of its page.
#include "pa_write.h"

namespace pa {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// E4M3 code of v: bit 7 sign, bits 6..3 exponent (bias 7), bits 2..0
// mantissa.  The nearest code value, ties to the even mantissa; magnitudes
// of 448 and more (infinity included) saturate to 448 (0x7E); NaN gives the
// NaN code s.1111.111.
__device__ __forceinline__ uint32_t e4m3_code(float v) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return sign | 0x7fu;   // NaN
  if (a >= 0x43e00000u) return sign | 0x7eu;  // |v| >= 448
  if (a < 0x3c800000u) {
    // |v| < 2^-6: the subnormal codes m 2^-9, m = 0..8 (8 is the smallest
    // normal, code 0x08); |v| * 512 is exact, rint rounds half to even
    return sign | (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
  }
  // normal: exponent e in 1..15, mantissa rounded from 23 to 3 bits (ties to
  // even); a carry out of the mantissa moves to the next exponent, and no
  // value below 448 rounds past code 0x7E
  const uint32_t e = (a >> 23) - 120u;
  const uint32_t m23 = a & 0x7fffffu;
  const uint32_t m3 = (m23 + 0x7ffffu + ((m23 >> 20) & 1u)) >> 20;
  return sign | ((e << 3) + m3);
}

// Codes of the 8 bf16 elements in the 4 words of `w`, each divided by
// `scale` in fp32 (correctly rounded), packed little-endian into 2 words.
__device__ __forceinline__ uint2 quantize8(const u32x4_t &w, float scale) {
  uint32_t out[2] = {0u, 0u};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lo = __uint_as_float(w[i] << 16);
    const float hi = __uint_as_float(w[i] & 0xffff0000u);
    const uint32_t c = e4m3_code(__fdiv_rn(lo, scale)) | (e4m3_code(__fdiv_rn(hi, scale)) << 8);
    out[i / 2] |= c << (16 * (i % 2));
  }
  return make_uint2(out[0], out[1]);
}

template <int LANES>
__global__ __launch_bounds__(256) void append_fp8_kernel(AppendParams p) {
  constexpr int kRowsPerBlock = 256 / LANES;
  const int part = threadIdx.x % LANES;  // 16-byte piece of the source row
  const long long rows = (long long)p.tokens * p.Hkv;
  const long long stride = (long long)gridDim.x * kRowsPerBlock;
  for (long long r = (long long)blockIdx.x * kRowsPerBlock + threadIdx.x / LANES; r < rows;
       r += stride) {
    const int t = (int)(r / p.Hkv);
    const int h = (int)(r - (long long)t * p.Hkv);
    const int s = p.slots[t];
    if (s < 0 || s >= p.num_slots) continue;
    const int page = s / p.ps;
    const int off = s - page * p.ps;
    const size_t src = (size_t)r * LANES + part;  // in 16-byte units
    const size_t dst = (((size_t)page * p.Hkv + h) * p.ps + off) * LANES + part;  // 8-byte units
    const u32x4_t kv = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p.k) + src);
    const u32x4_t vv = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p.v) + src);
    reinterpret_cast<uint2 *>(p.kp)[dst] = quantize8(kv, p.k_scale);
    reinterpret_cast<uint2 *>(p.vp)[dst] = quantize8(vv, p.v_scale);
  }
}

template <int LANES>
__global__ __launch_bounds__(256) void append_kernel(AppendParams p) {
  constexpr int kRowsPerBlock = 256 / LANES;
  const int part = threadIdx.x % LANES;  // 16-byte piece of the row
  const long long rows = (long long)p.tokens * p.Hkv;
  const long long stride = (long long)gridDim.x * kRowsPerBlock;
  for (long long r = (long long)blockIdx.x * kRowsPerBlock + threadIdx.x / LANES; r < rows;
       r += stride) {
    const int t = (int)(r / p.Hkv);
    const int h = (int)(r - (long long)t * p.Hkv);
    const int s = p.slots[t];
    if (s < 0 || s >= p.num_slots) continue;
    const int page = s / p.ps;
    const int off = s - page * p.ps;
    const size_t src = (size_t)r * LANES + part;  // in 16-byte units
    const size_t dst = (((size_t)page * p.Hkv + h) * p.ps + off) * LANES + part;
    const u32x4_t kv = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p.k) + src);
    const u32x4_t vv = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p.v) + src);
    reinterpret_cast<u32x4_t *>(p.kp)[dst] = kv;
    reinterpret_cast<u32x4_t *>(p.vp)[dst] = vv;
  }
}

template <int LANES>
hipError_t launch(const AppendParams &p, hipStream_t stream) {
  constexpr int kRowsPerBlock = 256 / LANES;
  const long long rows = (long long)p.tokens * p.Hkv;
  const long long want = (rows + kRowsPerBlock - 1) / kRowsPerBlock;
  const int blocks = (int)(want < 256 * 16 ? want : 256 * 16);  // grid-stride past 16 per CU
  if (p.fp8)
    hipLaunchKernelGGL((append_fp8_kernel<LANES>), dim3(blocks), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((append_kernel<LANES>), dim3(blocks), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_append(const AppendParams &p, hipStream_t stream) {
  if (p.row_bytes == 128) return launch<8>(p, stream);
  if (p.row_bytes == 256) return launch<16>(p, stream);
  return launch<32>(p, stream);
}

}  // namespace pa
