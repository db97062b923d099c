// Internal launch interface of the K/V write path (pa_append) between the
// C-ABI host layer (pa_host.cpp) and pa_append.hip.  Not installed; the
// public ABI is pa.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

// Scatter of token rows to page-pool slots, already validated by the host.
struct AppendParams {
  const void *k;
  const void *v;
  const int32_t *slots;
  void *kp;
  void *vp;
  int32_t tokens;
  int32_t Hkv;
  int32_t ps;
  int32_t num_slots;     // num_pages * page_size (< 2^31)
  int32_t row_bytes;     // head_dim * source element bytes: 128, 256 or 512
  int32_t fp8;           // 1: bf16 rows quantised into fp8 E4M3 pages
  float k_scale, v_scale;
};
hipError_t launch_append(const AppendParams &p, hipStream_t stream);

}  // namespace pa
