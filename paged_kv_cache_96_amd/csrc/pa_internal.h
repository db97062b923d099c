// Internal launch interface between the C-ABI host layer (pa_host.cpp) and
// the kernel translation units.  Not installed; the public ABI is pa.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

enum class DType { F32 = 0, BF16 = 1 };

// Everything a paged-attention launch needs, already validated by the host.
struct LaunchParams {
  const void *q;
  const void *kp;
  const void *vp;
  const int32_t *bt;
  const int32_t *cl;
  const int32_t *ql;        // nullptr: every request has L rows
  void *out;
  float *ws_o;              // partitions: [B, Hq, L, S, D]; balanced: [S, ROWS, D] fp32;
                            // prefill key split: [S, D / 8, 256, 4] (nullptr: no split)
  float *ws_lse;            // partitions: [B, Hq, L, S];    balanced: [S, ROWS]    fp32;
                            // prefill key split: [S, 2, 256]
  int32_t *dbg_trace;       // nullptr unless instrumented
  int32_t *dbg_visits;      // nullptr unless instrumented
  // Contract checks: nullptr, or the int32 [2] word the check kernel fills
  // before the call's kernels, which then return at once when dbg_errors[0]
  // is nonzero (debug_errors in pa.h).
  const int32_t *dbg_errors;
  uint32_t *counters;       // balanced: per row block arrival counters (fused merge), or nullptr
  int32_t B, Hq, Hkv, L, D, num_pages, ps, max_pages;
  int32_t causal;
  int32_t num_splits;       // S >= 1: partitions, or piece slots when balanced
  int32_t part_tokens;      // keys per partition, multiple of ps (partition schedule)
  int32_t balanced;         // 1: equal runs of steps per wave (see decode_balanced_waves)
  int32_t grid_waves;       // balanced: waves of the decode grid
  float scale_log2;         // scale * log2(e): scores are kept in base-2 units
  int32_t kv_fp8;           // 1: the pages hold fp8 E4M3 codes (query and out bf16)
  float k_scale, v_scale;   // fp8 pages: element value = code value * scale (else 1)
  const int32_t *qsl;       // packed rows: query_start_loc [B + 1], or nullptr ([B, Hq, L])
  int32_t num_tokens;       // packed rows: T = qsl[B] when the caller gives it, else 0
  int32_t route;            // 0: every request; ragged call: 1 its decode requests, 2 the rest
  // Shared prefixes (pa_decode_shared): request groups grp_start[k] ..
  // grp_start[k + 1] - 1 read the same first grp_pre[k] keys (rounded down to
  // whole pages).  Decode launch (prefix_pass 0): each request walks its keys
  // past the prefix and merges the prefix state of its rows.  Prefix launch
  // (prefix_pass 1, prefill kernel): virtual request k holds the query rows
  // of the members of group k (Lm rows each, member-major) over the prefix
  // keys of the group's first member, and writes each row's state.
  const int32_t *grp_start; // [num_groups + 1], or nullptr (no shared prefixes)
  const int32_t *grp_pre;   // [num_groups]
  int32_t num_groups;
  int32_t prefix_pass;
  int32_t Lm;               // prefix launch: query rows per member (the call's q_len)
  // Prefix states by output row: the prefix launch splits a group's prefix
  // keys into at most kPrefixPieces pieces per row tile, and piece s of a
  // row leaves its normalised output pre_o[(row * kPrefixPieces + s) * D ..]
  // and natural-log log-sum-exp pre_lse[row * kPrefixPieces + s] (-inf: no
  // key); pre_n[row] is the row's piece count.  The decode launch folds them
  // into the row's merge.
  float *pre_o;
  float *pre_lse;
  int32_t *pre_n;
};

// Most pieces the prefix launch cuts one row tile's prefix keys into (so a
// row's prefix states fit one batch of loads of the decode merge).
constexpr int kPrefixPieces = 16;

// Query rows of request b.
__device__ __forceinline__ int query_rows(const LaunchParams &p, int b) {
  return p.qsl ? p.qsl[b + 1] - p.qsl[b] : (p.ql ? p.ql[b] : p.L);
}

// Row index of query / output row (request b, head h, position i): packed
// rows [T, Hq] (T = qsl[B]) or padded [B, Hq, L].
__device__ __forceinline__ size_t query_row(const LaunchParams &p, int b, int h, int i) {
  return p.qsl ? (size_t)(p.qsl[b] + i) * p.Hq + h : ((size_t)b * p.Hq + h) * p.L + i;
}

// Shared keys of group k: its prefix length rounded down to whole pages
// (only whole pages are shared), within [0, max_pages * page_size] (so a
// length beyond the contract never reads past a block-table row).
__device__ __forceinline__ int group_prefix_keys(const LaunchParams &p, int k) {
  const int n = min(p.grp_pre[k], p.max_pages * p.ps);
  return n > 0 ? n - n % p.ps : 0;
}

// Whether a request of Lb query rows takes the decode route of a ragged
// call: one query row (or none) and a GQA group that one decode row block
// holds.  Every other request takes the prefill route.
__host__ __device__ inline bool ragged_decode_request(int G, int Lb) { return G <= 8 && Lb <= 1; }

// Whether request b belongs to this launch.
__device__ __forceinline__ bool routed_here(const LaunchParams &p, int Lb) {
  if (p.route == 0) return true;
  return (p.route == 1) == ragged_decode_request(p.Hq / p.Hkv, Lb);
}

// Whether the call's contract check found a violation: then a kernel of the
// call reads no block-table entry and K/V element and writes nothing.  One
// wave-uniform branch on a kernel argument when no check runs.
__device__ __forceinline__ bool contract_broken(const LaunchParams &p) {
  return p.dbg_errors != nullptr && p.dbg_errors[0] != 0;
}

// The contract check of a call (pa_validate.hip): checks on the device every
// block-table entry the call's kernels would read, the context lengths, the
// query rows and (max_group > 0) the shared-prefix groups, and ORs PA_DEBUG_*
// flags into errors[0] and adds the count of bad entries to errors[1].
hipError_t launch_validate(const LaunchParams &p, int32_t *errors, int max_group,
                           hipStream_t stream);

// Vector-ALU paged decode kernel (also the fp32 prefill path, with S == 1).
hipError_t launch_decode(const LaunchParams &p, DType dt, hipStream_t stream);
// Log-sum-exp merge of decode partitions into `out`.
hipError_t launch_split_reduce(const LaunchParams &p, DType dt, hipStream_t stream);
// bf16 MFMA prefill kernel.
hipError_t launch_prefill_mfma(const LaunchParams &p, hipStream_t stream);

// Largest batch the balanced decode schedule supports (its per-request
// prefix sums live in LDS); larger batches use the partition schedule.
constexpr int kBalancedMaxBatch = 2048;
// Bound on the total number of steps of a balanced call, so that products of
// a step index and a wave count stay far inside 64 bits.
constexpr int64_t kBalancedMaxSteps = int64_t(1) << 40;
// Bound on (row blocks of the call) x (steps of the call) for the balanced
// schedule, so that the wave cap's product kBalancedWaveFactor * units * T
// fits in 64 bits.
constexpr int64_t kBalancedMaxUnitSteps = int64_t(1) << 60;
// Shortest run of steps a balanced schedule hands to one wave.
constexpr int kBalancedMinSteps = 4;
// Setup cost of a row block in the balanced schedule, in steps: a wave that
// starts a new row block inside its run pays the previous piece's write and
// arrival and the new piece's block-table, query and first K/V latencies
// (measured ~6-7 us, ~5 steps of 1.25 us, on C2-like calls).  Every row
// block with keys is laid out as kUnitSetupSteps setup positions followed
// by its steps, so runs are equal in cost rather than in steps.
constexpr int kUnitSetupSteps = 5;
// Cap on the waves of a balanced call over `units` row blocks and T steps:
// Wa^2 <= kBalancedWaveFactor * units * T.  With p = Wa / units pieces per row
// block and s = T / Wa steps per run, that is s >= p / kBalancedWaveFactor: a
// small batch over long contexts is no longer cut into 100+ pieces of a few
// steps per row block, whose per-piece costs (setup, state write, merge read)
// outweigh the extra waves.  Measured best near s = p / 4 for 1-2 requests
// over 4k-32k keys; large batches are bounded by the slot count first.
constexpr int kBalancedWaveFactor = 4;

// floor(sqrt(x)) for x >= 0, exact on host and device.
__host__ __device__ inline int64_t isqrt64(int64_t x) {
  if (x < 2) return x;
  int64_t r = (int64_t)sqrt((double)x);
  while (r * r > x) --r;
  while ((r + 1) * (r + 1) <= x) ++r;
  return r;
}

// Largest number of (request, tile) pairs the key split of the bf16 prefill
// plans over (the plan's tables live in the kernel's staging buffers);
// larger calls run unsplit.
constexpr int kSplitMaxPairs = 2048;

// Keys per decode step (one 16-byte load per lane, four loads per step):
// 16 for bf16 with D = 128, 32 for fp8 pages with D = 128.  elem_bytes is
// the byte size of a page element.
__host__ __device__ constexpr int decode_step_keys(int D, int elem_bytes) {
  return 4096 / (D * elem_bytes);
}

// Waves of the balanced decode grid for `p` (the resident capacity of the
// kernel variant that would run it).
int decode_balanced_waves(const LaunchParams &p, DType dt);

// How a balanced call splits its T steps: wave v < Wa owns the steps
// [begin(v), begin(v + 1)), equal shares in step order.  The piece of row
// block r (counted over the call) walked by wave v lives in slot r + v: row
// blocks and waves' runs are both consecutive intervals of the step order,
// so a later row block never meets an earlier wave and r + v is unique;
// slots stay below units + Wa.
struct BalancedSplit {
  int64_t T = 0, Wa = 0;
  __host__ __device__ int64_t begin(int64_t v) const { return Wa > 0 ? v * T / Wa : 0; }
  // wave of step t < T: the largest v with begin(v) <= t
  __host__ __device__ int64_t wave_of(int64_t t) const { return ((t + 1) * Wa - 1) / T; }
};

__host__ __device__ inline BalancedSplit balanced_split(int64_t grid_waves, int64_t T, int64_t units,
                                                        int64_t S) {
  BalancedSplit s;
  s.T = T;
  if (T <= 0) return s;
  int64_t w = grid_waves;
  const int64_t by_len = (T + kBalancedMinSteps - 1) / kBalancedMinSteps;
  if (by_len < w) w = by_len;
  // kBalancedWaveFactor * units * T stays below 2^63 (the host keeps units *
  // T <= 2^60); were it larger, its root would exceed any grid anyway
  if (units <= (INT64_MAX / kBalancedWaveFactor) / T) {
    const int64_t by_pieces = isqrt64(kBalancedWaveFactor * units * T);
    if (by_pieces < w) w = by_pieces;
  }
  if (S - units < w) w = S - units;  // S >= units + 1 is checked by the host
  s.Wa = w;
  return s;
}

// Query rows one decode workgroup holds, for a GQA group of `rows_per_head`
// packed rows (G * L).  Shared by the host (grid sizing) and the launcher.
__host__ __device__ inline int decode_rows_per_block(int rows) {
  if (rows <= 1) return 1;
  if (rows <= 2) return 2;
  if (rows <= 4) return 4;
  return 8;
}

}  // namespace pa
