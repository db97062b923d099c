// Log-sum-exp merge of split-KV partition states ("Reading vLLM's
// PagedAttention Kernel", section 3.3: partitions computed in parallel are
// combined afterwards).  One wave per query row:
//   M = max_s lse_s,  w_s = exp(lse_s - M),  out = sum_s w_s o_s / sum_s w_s
// over the partitions s < ceil(ctx / partition_tokens) that the decode
// kernel wrote.  Rows past query_lens[b], and requests with no keys, get 0.
#include "pa_common.hpp"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr float kLog2e = 1.44269504088896340736f;

template <typename T, int D>
__global__ __launch_bounds__(256) void split_reduce_kernel(LaunchParams p, int total_rows) {
  constexpr int kPer = D / 64;  // output elements per lane
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= total_rows) return;
  const int i = row % p.L;
  const int b = row / (p.L * p.Hq);
  const int ctx = p.cl[b];
  const int Lb = p.ql ? p.ql[b] : p.L;
  const int S = p.num_splits;
  const int n = (i < Lb && ctx > 0) ? min(S, (ctx + p.part_tokens - 1) / p.part_tokens) : 0;

  const float *lse = p.ws_lse + (size_t)row * S;
  const float *po = p.ws_o + (size_t)row * S * D;
  float M = kNegInf;
  for (int s = lane; s < n; s += 64) M = fmaxf(M, lse[s]);
  M = group_max<64>(M);

  float o[kPer];
#pragma unroll
  for (int e = 0; e < kPer; ++e) o[e] = 0.f;
  if (M != kNegInf) {
    float wsum = 0.f;
    for (int s = 0; s < n; ++s) {
      const float w = fast_exp2((lse[s] - M) * kLog2e);
      wsum += w;
#pragma unroll
      for (int e = 0; e < kPer; ++e) o[e] = fmaf(w, po[(size_t)s * D + e * 64 + lane], o[e]);
    }
    const float inv = 1.f / wsum;
#pragma unroll
    for (int e = 0; e < kPer; ++e) o[e] *= inv;
  }
  T *out = reinterpret_cast<T *>(p.out) + (size_t)row * D;
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    if constexpr (sizeof(T) == 4) {
      out[e * 64 + lane] = o[e];
    } else {
      out[e * 64 + lane] = (uint16_t)f32_to_bf16(o[e]);
    }
  }
}

template <typename T, int D>
hipError_t launch(const LaunchParams &p, hipStream_t stream) {
  const int rows = p.B * p.Hq * p.L;
  hipLaunchKernelGGL((split_reduce_kernel<T, D>), dim3((rows + 3) / 4), dim3(256), 0, stream, p,
                     rows);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_split_reduce(const LaunchParams &p, DType dt, hipStream_t stream) {
  if (dt == DType::F32) return p.D == 64 ? launch<float, 64>(p, stream) : launch<float, 128>(p, stream);
  return p.D == 64 ? launch<uint16_t, 64>(p, stream) : launch<uint16_t, 128>(p, stream);
}

}  // namespace pa
