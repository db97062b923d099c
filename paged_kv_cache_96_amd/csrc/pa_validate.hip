// Contract check of a call (debug mode): the library's kernels take block
// tables, context lengths and query rows on trust ("Week 3 Day 4: Direct
// Paged Attention", "What Must Hold, and What Breaks If It Doesn't": a page
// id outside the pool or a context longer than the table reads memory that
// is not the request's).  With pa_args.debug_errors set, this kernel runs
// first on the call's stream and reads only the metadata, never K/V:
//
//   PA_DEBUG_BAD_CONTEXT  context_lens[b] < 0 or > max_pages * page_size;
//   PA_DEBUG_BAD_PAGE     an entry block_table[b][j], j < ceil(ctx_b /
//                         page_size) (the entries the kernels read; ctx_b
//                         clamped to the table), outside [0, num_pages);
//                         errors[1] counts these entries;
//   PA_DEBUG_BAD_ROWS     query rows of a request outside [0, q_len]
//                         (query_lens, or query_start_loc not starting at 0
//                         and nondecreasing), or a causal request with keys
//                         but more query rows than keys;
//   PA_DEBUG_BAD_GROUPS   shared prefixes: group_start not 0 .. nondecreasing
//                         .. <= batch, a group larger than max_group_size, a
//                         negative prefix length, a member whose keys before
//                         its query rows do not cover the group's shared keys,
//                         or a member whose table differs from the first
//                         member's on the shared pages.
//
// The flags are ORed into errors[0]; every kernel of the call reads
// errors[0] first and returns when it is nonzero (contract_broken).
#include "pa_internal.h"
#include "pa.h"

namespace pa {
namespace {

__device__ __forceinline__ int rows_of(const LaunchParams &p, int b, bool &bad) {
  int r;
  if (p.qsl) {
    const int lo = p.qsl[b], hi = p.qsl[b + 1];
    if (b == 0 && lo != 0) bad = true;
    r = hi - lo;
  } else {
    r = p.ql ? p.ql[b] : p.L;
  }
  if (r < 0 || r > p.L) bad = true;
  return r;
}

// Group of request b: the largest k with grp_start[k] <= b (the starts need
// not be valid: every probe stays inside [0, num_groups]); -1 if none.
__device__ __forceinline__ int group_of(const LaunchParams &p, int b) {
  if (p.num_groups <= 0 || b < p.grp_start[0] || b >= p.grp_start[p.num_groups]) return -1;
  int lo = 0, hi = p.num_groups - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (p.grp_start[mid] <= b) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__global__ __launch_bounds__(256) void validate_kernel(LaunchParams p, int32_t *errors,
                                                       int max_group) {
  __shared__ int s_flags, s_bad;
  if (threadIdx.x == 0) s_flags = s_bad = 0;
  __syncthreads();
  int flags = 0, bad = 0;
  const long long cap = (long long)p.max_pages * p.ps;
  const long long n = (long long)p.B * p.max_pages;
  const long long stride = (long long)gridDim.x * blockDim.x;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    const int b = (int)(i / p.max_pages);
    const int j = (int)(i - (long long)b * p.max_pages);
    const int ctx = p.cl[b];
    const long long cc = ctx < 0 ? 0 : (ctx > cap ? cap : ctx);
    if (j < (cc + p.ps - 1) / p.ps) {
      const int page = p.bt[i];
      if (page < 0 || page >= p.num_pages) {
        flags |= PA_DEBUG_BAD_PAGE;
        ++bad;
      }
    }
    int k = -1;
    if (max_group > 0) k = group_of(p, b);
    if (j == 0) {
      if (ctx < 0 || ctx > cap) flags |= PA_DEBUG_BAD_CONTEXT;
      bool bad_rows = false;
      const int r = rows_of(p, b, bad_rows);
      // (an empty context is the zero-output case, not a violation)
      if (bad_rows || (p.causal && ctx > 0 && r > ctx)) flags |= PA_DEBUG_BAD_ROWS;
      if (k >= 0 && (long long)ctx - r < group_prefix_keys(p, k)) flags |= PA_DEBUG_BAD_GROUPS;
    }
    if (k >= 0) {
      const int first = p.grp_start[k];  // in [0, b] when the starts are valid
      if (first < 0 || first >= p.B) {
        flags |= PA_DEBUG_BAD_GROUPS;
      } else if (b != first && j < group_prefix_keys(p, k) / p.ps &&
          p.bt[(long long)first * p.max_pages + j] != p.bt[i])
        flags |= PA_DEBUG_BAD_GROUPS;
    }
  }
  if (max_group > 0) {
    // group structure: starts 0 .. nondecreasing .. <= B, sizes, prefixes
    for (long long k = (long long)blockIdx.x * blockDim.x + threadIdx.x; k <= p.num_groups;
         k += stride) {
      const int s = p.grp_start[k];
      if (k == 0 && s != 0) flags |= PA_DEBUG_BAD_GROUPS;
      if (k == p.num_groups && s > p.B) flags |= PA_DEBUG_BAD_GROUPS;
      if (k < p.num_groups) {
        const int e = p.grp_start[k + 1];
        if (e < s || e - s > max_group || p.grp_pre[k] < 0) flags |= PA_DEBUG_BAD_GROUPS;
      }
    }
  }
  if (flags) atomicOr(&s_flags, flags);
  if (bad) atomicAdd(&s_bad, bad);
  __syncthreads();
  if (threadIdx.x == 0) {
    if (s_flags) atomicOr(errors, s_flags);
    if (s_bad) atomicAdd(errors + 1, s_bad);
  }
}

}  // namespace

hipError_t launch_validate(const LaunchParams &p, int32_t *errors, int max_group,
                           hipStream_t stream) {
  const long long n = (long long)p.B * p.max_pages;
  const long long g = max_group > 0 && p.num_groups + 1 > n ? p.num_groups + 1 : n;
  const unsigned blocks = (unsigned)(g / 256 + 1 < 1024 ? g / 256 + 1 : 1024);
  hipLaunchKernelGGL(validate_kernel, dim3(blocks), dim3(256), 0, stream, p, errors, max_group);
  return hipGetLastError();
}

}  // namespace pa
