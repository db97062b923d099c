// Internal launch interface between the C-ABI host layer (pa_host.cpp) and
// the kernel translation units.  Not installed; the public ABI is pa.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

// Everything a paged-attention launch needs, already validated by the host.
struct LaunchParams {
  const void *q;
  const void *kp;
  const void *vp;
  const int32_t *bt;
  const int32_t *cl;
  const int32_t *ql;        // nullptr: every request has L rows
  void *out;
  float *ws_o;              // [B, Hq, L, S, D] fp32 (decode with S > 1)
  float *ws_lse;            // [B, Hq, L, S]   fp32
  int32_t *dbg_trace;       // nullptr unless instrumented
  int32_t *dbg_visits;      // nullptr unless instrumented
  uint32_t *counters;       // decode work-queue counters [2], or nullptr (plain grid)
  int32_t B, Hq, Hkv, L, D, num_pages, ps, max_pages;
  int32_t causal;
  int32_t num_splits;       // S >= 1
  int32_t part_tokens;      // keys per partition, multiple of ps
  float scale_log2;         // scale * log2(e): scores are kept in base-2 units
};

enum class DType { F32 = 0, BF16 = 1 };

// Vector-ALU paged decode kernel (also the fp32 prefill path, with S == 1).
hipError_t launch_decode(const LaunchParams &p, DType dt, hipStream_t stream);
// Log-sum-exp merge of decode partitions into `out`.
hipError_t launch_split_reduce(const LaunchParams &p, DType dt, hipStream_t stream);
// bf16 MFMA prefill kernel.
hipError_t launch_prefill_mfma(const LaunchParams &p, hipStream_t stream);

// Largest batch the persistent decode schedule supports (its per-request
// partition counts live in LDS); larger batches use the plain grid.
constexpr int kDecodeQueueMaxBatch = 2048;

// Query rows one decode workgroup holds, for a GQA group of `rows_per_head`
// packed rows (G * L).  Shared by the host (grid sizing) and the launcher.
inline int decode_rows_per_block(int rows) {
  if (rows <= 1) return 1;
  if (rows <= 2) return 2;
  if (rows <= 4) return 4;
  return 8;
}

}  // namespace pa
