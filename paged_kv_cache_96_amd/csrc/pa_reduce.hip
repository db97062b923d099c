// Log-sum-exp merge of split-KV partition states ("Reading vLLM's
// PagedAttention Kernel", section 3.3: partitions computed in parallel are
// combined afterwards).  One wave per query row:
//   M = max_s lse_s,  w_s = exp(lse_s - M),  out = sum_s w_s o_s / sum_s w_s
// over the states the decode kernel wrote: partitions s < ceil(ctx /
// partition_tokens) under the partition schedule; under the balanced
// schedule the pieces w0..w1 of the row block, recomputed from the same
// formula the decode kernel used (a row block that one wave covered was
// written by the decode kernel and is left alone).  Rows past query_lens[b],
// and requests with no keys, get 0.
#include "pa_common.hpp"
#include "pa_internal.h"
#include "pa_merge.hpp"

namespace pa {
namespace {

// Sum over the 64 lanes of a wave.
__device__ __forceinline__ long long wave_sum(long long v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Waves w0..w1 of the balanced decode schedule that walked unit u of
// request b (units per request); count 0 when the request has no keys.
template <int kStep>
__device__ void balanced_waves(const LaunchParams &p, int b, int u, int units, long long &w0,
                               int &count) {
  const int lane = threadIdx.x & 63;
  long long tot = 0, before = 0;
  for (int c = lane; c < p.B; c += 64) {
    // requests of another route have no steps (as in the decode kernel)
    const int ctx = routed_here(p, query_rows(p, c)) ? p.cl[c] : 0;
    const long long n = (ctx + kStep - 1) / kStep;
    const long long steps = (long long)units * (n > 0 ? n + kUnitSetupSteps : 0);
    tot += steps;
    if (c < b) before += steps;
  }
  tot = wave_sum(tot);
  before = wave_sum(before);
  const long long n = (p.cl[b] + kStep - 1) / kStep;
  w0 = 0;
  count = 0;
  if (n == 0) return;
  const BalancedSplit bs = balanced_split(p.grid_waves, tot, (long long)p.B * units, p.num_splits);
  const long long row0 = before + (long long)u * (n + kUnitSetupSteps) + kUnitSetupSteps;
  w0 = bs.wave_of(row0);
  count = (int)(bs.wave_of(row0 + n - 1) - w0 + 1);
}

// KVB: bytes of a page element (the decode step, and so the balanced split,
// depends on it).
template <typename T, int D, int KVB>
__global__ __launch_bounds__(256) void split_reduce_kernel(LaunchParams p, int total_rows) {
  if (contract_broken(p)) return;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= total_rows) return;
  const int i = row % p.L;
  const int b = row / (p.L * p.Hq);
  const int ctx = p.cl[b];
  const int Lb = query_rows(p, b);
  if (!routed_here(p, Lb)) return;
  if (p.qsl && i >= Lb) return;  // packed rows: no padding rows exist
  // this row's index in the output (and in the partition states)
  const size_t orow = query_row(p, b, (row / p.L) % p.Hq, i);
  const int S = p.num_splits;
  int n;
  // state s of this row: lse[s * stride], po[s * stride * D]
  const float *lse;
  const float *po;
  size_t stride;
  if (p.balanced) {
    const int h = (row / p.L) % p.Hq;
    const int G = p.Hq / p.Hkv;
    const int g = h / G;
    const int rows = decode_rows_per_block(G * p.L);
    const int row_blocks = (G * p.L + rows - 1) / rows;
    const int rho = i * G + (h - g * G);
    const int u = g * row_blocks + rho / rows;
    long long w0;
    int pieces;
    balanced_waves<decode_step_keys(D, KVB)>(p, b, u, p.Hkv * row_blocks, w0, pieces);
    if (pieces == 1) return;  // the decode kernel wrote this row
    n = i < Lb ? pieces : 0;
    const size_t first = ((size_t)b * p.Hkv * row_blocks + u + w0) * rows + rho % rows;
    lse = p.ws_lse + first;
    po = p.ws_o + first * D;
    stride = rows;
  } else {
    n = (i < Lb && ctx > 0) ? min(S, (ctx + p.part_tokens - 1) / p.part_tokens) : 0;
    lse = p.ws_lse + orow * S;
    po = p.ws_o + orow * S * D;
    stride = 1;
  }

  merge_row<T, D>(lse, po, (int)stride, n, reinterpret_cast<T *>(p.out) + orow * D);
}

template <typename T, int D, int KVB = (int)sizeof(T)>
hipError_t launch(const LaunchParams &p, hipStream_t stream) {
  const int rows = p.B * p.Hq * p.L;
  hipLaunchKernelGGL((split_reduce_kernel<T, D, KVB>), dim3((rows + 3) / 4), dim3(256), 0, stream,
                     p, rows);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_split_reduce(const LaunchParams &p, DType dt, hipStream_t stream) {
  if (dt == DType::F32) return p.D == 64 ? launch<float, 64>(p, stream) : launch<float, 128>(p, stream);
  if (p.kv_fp8) return launch<uint16_t, 128, 1>(p, stream);  // fp8 pages: D = 128 only
  return p.D == 64 ? launch<uint16_t, 64>(p, stream) : launch<uint16_t, 128>(p, stream);
}

}  // namespace pa
