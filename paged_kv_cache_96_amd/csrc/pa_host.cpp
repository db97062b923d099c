// C-ABI host layer of libpa.so: synchronous validation, the split plan, and
// kernel launches on the caller's stream.  Nothing here allocates device
// memory or synchronises.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <mutex>

#include <hip/hip_runtime.h>

#include "pa.h"
#include "pa_internal.h"
#include "pa_write.h"

#define PA_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

constexpr int kMinPartitionTokens = 256;  // below this the merge costs more than it buys
constexpr int kBlocksPerCu = 8;           // decode work items wanted per compute unit
constexpr int kWavesPerCu = 4;            // balanced decode: active waves per compute unit
                                          // (one per SIMD keeps enough loads in flight and
                                          // halves the pieces to merge; measured faster)
constexpr int kMaxGridYZ = 65535;

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Size checks shared by every entry point (no pointer is dereferenced).
pa_status check_sizes(const pa_args *a) {
  if (!a) return PA_ERR_INVALID_ARG;
  if (a->batch < 0 || a->num_q_heads < 1 || a->num_kv_heads < 1 || a->q_len < 1 ||
      a->head_dim < 1 || a->num_pages < 1 || a->page_size < 1 || a->max_pages < 1)
    return PA_ERR_INVALID_ARG;
  if (a->num_q_heads % a->num_kv_heads != 0) return PA_ERR_INVALID_ARG;
  if (a->mask != PA_MASK_NONE && a->mask != PA_MASK_CAUSAL) return PA_ERR_INVALID_ARG;
  if (!(a->scale > 0.f) || !isfinite(a->scale)) return PA_ERR_INVALID_ARG;
  if ((int64_t)a->max_pages * a->page_size > INT32_MAX / 2) return PA_ERR_INVALID_ARG;
  if (a->batch > kMaxGridYZ) return PA_ERR_INVALID_ARG;
  if (a->dtype != PA_DTYPE_F32 && a->dtype != PA_DTYPE_BF16) return PA_ERR_UNSUPPORTED;
  if (a->head_dim != 64 && a->head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (a->query_start_loc && a->query_lens) return PA_ERR_INVALID_ARG;  // one or the other
  if (a->num_tokens < 0 ||
      (a->query_start_loc && (int64_t)a->num_tokens > (int64_t)a->batch * a->q_len))
    return PA_ERR_INVALID_ARG;
  if (a->kv_dtype != PA_KV_SAME && a->kv_dtype != PA_KV_FP8_E4M3) return PA_ERR_INVALID_ARG;
  if (a->kv_dtype == PA_KV_FP8_E4M3) {
    if (!(a->k_scale > 0.f) || !isfinite(a->k_scale) || !(a->v_scale > 0.f) ||
        !isfinite(a->v_scale))
      return PA_ERR_INVALID_ARG;
    if (a->dtype != PA_DTYPE_BF16 || a->head_dim != 128) return PA_ERR_UNSUPPORTED;
  }
  return PA_OK;
}

bool kv_fp8(const pa_args *a) { return a->kv_dtype == PA_KV_FP8_E4M3; }

// A call with nothing to compute: no requests, or packed rows with no row at
// all (T = 0), which the caller states by passing NULL query and out.
bool nothing_to_do(const pa_args *a) {
  return a->batch == 0 || (a->query_start_loc && !a->query && !a->out);
}

pa_status check_pointers(const pa_args *a) {
  if (!a->query || !a->key_pages || !a->value_pages || !a->block_table || !a->context_lens ||
      !a->out)
    return PA_ERR_INVALID_ARG;
  if (!aligned16(a->query) || !aligned16(a->key_pages) || !aligned16(a->value_pages) ||
      !aligned16(a->out))
    return PA_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(a->debug_errors) & 3u) return PA_ERR_INVALID_ARG;
  return PA_OK;
}

// The contract check of a call, enqueued before its kernels when the caller
// asks for it (pa_args.debug_errors); `groups` for pa_decode_shared.
pa_status enqueue_check(const pa_args *a, const pa_prefix_groups *groups, hipStream_t stream) {
  if (!a->debug_errors) return PA_OK;
  pa::LaunchParams p;
  memset(&p, 0, sizeof p);
  p.bt = a->block_table;
  p.cl = a->context_lens;
  p.ql = a->query_lens;
  p.qsl = a->query_start_loc;
  p.B = a->batch;
  p.L = a->q_len;
  p.num_pages = a->num_pages;
  p.ps = a->page_size;
  p.max_pages = a->max_pages;
  p.causal = a->mask == PA_MASK_CAUSAL;
  int max_group = 0;
  if (groups) {
    p.grp_start = groups->group_start;
    p.grp_pre = groups->prefix_lens;
    p.num_groups = groups->num_groups;
    max_group = groups->max_group_size;
  }
  return pa::launch_validate(p, a->debug_errors, max_group, stream) == hipSuccess ? PA_OK
                                                                                 : PA_ERR_HIP;
}

// Bytes of one page element (the decode step depends on it).
int elem_bytes(const pa_args *a) {
  return kv_fp8(a) ? 1 : a->dtype == PA_DTYPE_F32 ? 4 : 2;
}

// Query rows of one decode row block.
int64_t decode_block_rows(const pa_args *a) {
  const int64_t rows = (int64_t)(a->num_q_heads / a->num_kv_heads) * a->q_len;
  return pa::decode_rows_per_block((int)(rows < 8 ? rows : 8));
}

// Row blocks (units of the decode schedule) per request.
int64_t decode_units(const pa_args *a) {
  const int64_t rows = (int64_t)(a->num_q_heads / a->num_kv_heads) * a->q_len;
  const int64_t per = decode_block_rows(a);
  return (int64_t)a->num_kv_heads * ((rows + per - 1) / per);
}

// a * b for a, b >= 0, saturating at INT64_MAX.
int64_t sat_mul(int64_t a, int64_t b) {
  return (b != 0 && a > INT64_MAX / b) ? INT64_MAX : a * b;
}

// Largest step count a balanced call over `a` can have (saturating).
int64_t balanced_max_steps(const pa_args *a) {
  const int64_t step = pa::decode_step_keys(a->head_dim, elem_bytes(a));
  const int64_t cap = (int64_t)a->max_pages * a->page_size;
  return sat_mul(sat_mul((int64_t)a->batch, decode_units(a)),
                 (cap + step - 1) / step + pa::kUnitSetupSteps);
}

// Whether the balanced schedule can serve `a`: batch, total steps and the
// product of row blocks and steps (the wave cap's operand) within bounds.
bool balanced_fits(const pa_args *a) {
  if (a->batch > pa::kBalancedMaxBatch) return false;
  const int64_t T = balanced_max_steps(a);
  if (T > pa::kBalancedMaxSteps) return false;
  const int64_t units = (int64_t)(a->batch > 0 ? a->batch : 1) * decode_units(a);
  return T == 0 || units <= pa::kBalancedMaxUnitSteps / T;
}

// Workspace consistency for a decode/merge pair.  A single partition needs
// no buffers.
pa_status check_workspace(const pa_args *a, const pa_workspace *ws, int32_t *S, int32_t *P,
                          bool *balanced) {
  const int32_t cap = a->max_pages * a->page_size;
  *balanced = false;
  if (ws && ws->schedule != PA_SCHEDULE_PARTITIONS && ws->schedule != PA_SCHEDULE_BALANCED)
    return PA_ERR_WORKSPACE;
  if (!ws || (ws->schedule == PA_SCHEDULE_PARTITIONS && ws->num_splits == 1)) {
    *S = 1;
    *P = cap;
    return PA_OK;
  }
  if (ws->schedule == PA_SCHEDULE_BALANCED) {
    // one piece slot per row block plus at least one wave
    if (!balanced_fits(a) || (int64_t)ws->num_splits < (int64_t)a->batch * decode_units(a) + 1)
      return PA_ERR_WORKSPACE;
    *balanced = true;
    *P = 0;
  } else {
    if (ws->num_splits < 1 || ws->partition_tokens <= 0 || ws->partition_tokens % a->page_size)
      return PA_ERR_WORKSPACE;
    if ((int64_t)ws->num_splits * ws->partition_tokens < cap) return PA_ERR_WORKSPACE;
    if (ws->num_splits > kMaxGridYZ) return PA_ERR_WORKSPACE;
    *P = ws->partition_tokens;
  }
  if (!ws->partial_out || !ws->partial_lse || !aligned16(ws->partial_out) ||
      !aligned16(ws->partial_lse))
    return PA_ERR_WORKSPACE;
  if (ws->counters && (!*balanced || (int64_t)ws->num_counters < (int64_t)a->batch * decode_units(a) ||
                       (reinterpret_cast<uintptr_t>(ws->counters) & 3u)))
    return PA_ERR_WORKSPACE;
  *S = ws->num_splits;
  return PA_OK;
}

pa::LaunchParams make_params(const pa_args *a, int32_t S, int32_t P, bool balanced,
                             const pa_workspace *ws) {
  pa::LaunchParams p;
  memset(&p, 0, sizeof p);
  p.q = a->query;
  p.kp = a->key_pages;
  p.vp = a->value_pages;
  p.bt = a->block_table;
  p.cl = a->context_lens;
  p.ql = a->query_lens;
  p.out = a->out;
  p.ws_o = (S > 1 && ws) ? ws->partial_out : nullptr;
  p.ws_lse = (S > 1 && ws) ? ws->partial_lse : nullptr;
  p.dbg_trace = a->debug_trace;
  p.dbg_visits = a->debug_visits;
  p.dbg_errors = a->debug_errors;
  p.counters = (balanced && ws) ? ws->counters : nullptr;
  p.B = a->batch;
  p.Hq = a->num_q_heads;
  p.Hkv = a->num_kv_heads;
  p.L = a->q_len;
  p.D = a->head_dim;
  p.num_pages = a->num_pages;
  p.ps = a->page_size;
  p.max_pages = a->max_pages;
  p.causal = a->mask == PA_MASK_CAUSAL;
  p.num_splits = S;
  p.part_tokens = P;
  p.balanced = balanced ? 1 : 0;
  p.grid_waves = 0;
  p.scale_log2 = a->scale * 1.4426950408889634f;
  p.kv_fp8 = kv_fp8(a) ? 1 : 0;
  p.k_scale = kv_fp8(a) ? a->k_scale : 1.f;
  p.v_scale = kv_fp8(a) ? a->v_scale : 1.f;
  p.qsl = a->query_start_loc;
  p.num_tokens = a->query_start_loc ? a->num_tokens : 0;
  p.route = 0;
  if (balanced) p.grid_waves = pa::decode_balanced_waves(p, (pa::DType)a->dtype);
  return p;
}

pa_status hip_status(hipError_t e) { return e == hipSuccess ? PA_OK : PA_ERR_HIP; }

// Workspace slots a launch uses (0 without a workspace).
int64_t ws_slots(const pa::LaunchParams &p) { return p.ws_o ? p.num_splits : 0; }

// Grid limits of the vector kernel under the partition schedule: gridDim.x =
// ceil(H_kv * row blocks * partitions / 4) (one work item per wave),
// gridDim.y = batch.
pa_status check_decode_grid(const pa_args *a, int32_t S) {
  const int64_t items = decode_units(a) * S;
  return (items + 3) / 4 > INT32_MAX ? PA_ERR_INVALID_ARG : PA_OK;
}

}  // namespace

PA_EXPORT int32_t pa_abi_version(void) { return PA_ABI_VERSION; }

PA_EXPORT const char *pa_status_string(int32_t status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_INVALID_ARG: return "invalid argument";
    case PA_ERR_UNSUPPORTED: return "unsupported head_dim or dtype";
    case PA_ERR_WORKSPACE: return "split workspace missing or inconsistent";
    case PA_ERR_HIP: return "HIP runtime error";
    case PA_ERR_SCRATCH:
      return "call needs more than the library scratch of pa_decode_noalloc holds";
    default: return "unknown status";
  }
}

PA_EXPORT pa_status pa_decode_plan(const pa_args *args, int32_t num_cus, pa_workspace *plan,
                                   size_t *workspace_bytes) {
  pa_status st = check_sizes(args);
  if (st != PA_OK) return st;
  if (!plan) return PA_ERR_INVALID_ARG;
  if (args->q_len > 8) return PA_ERR_INVALID_ARG;
  const int32_t ps = args->page_size;
  const int32_t cap = args->max_pages * ps;
  const int cus = num_cus > 0 ? num_cus : 256;
  const int64_t units = (int64_t)(args->batch > 0 ? args->batch : 1) * decode_units(args);
  int32_t S, P;
  if (plan->partition_tokens <= 0 && balanced_fits(args)) {
    // a piece slot per row block plus one per wave of the grid
    const int64_t slots = units + (int64_t)kWavesPerCu * cus;
    if (slots > INT32_MAX) return PA_ERR_INVALID_ARG;
    S = (int32_t)slots;
    P = 0;
    plan->schedule = PA_SCHEDULE_BALANCED;
    plan->num_counters = (int32_t)units;  // one arrival counter per row block
  } else {
    if (plan->partition_tokens > 0) {
      P = (plan->partition_tokens + ps - 1) / ps * ps;
    } else {
      const int64_t want = (int64_t)kBlocksPerCu * cus;
      const int64_t splits = units >= want ? 1 : (want + units - 1) / units;
      int64_t tok = (cap + splits - 1) / splits;
      if (tok < kMinPartitionTokens) tok = kMinPartitionTokens;
      P = (int32_t)((tok + ps - 1) / ps * ps);
    }
    if (P > cap) P = (cap + ps - 1) / ps * ps;
    if ((cap + P - 1) / P > kMaxGridYZ) {  // bounds the partition count
      const int64_t tok = ((int64_t)cap + kMaxGridYZ - 1) / kMaxGridYZ;
      P = (int32_t)((tok + ps - 1) / ps * ps);
    }
    S = (cap + P - 1) / P;
    plan->schedule = PA_SCHEDULE_PARTITIONS;
    plan->num_counters = 0;
  }
  plan->num_splits = S;
  plan->partition_tokens = P;
  if (workspace_bytes) {
    // partitions: [B, H_q, L, S] states; balanced: [S, rows per block] states
    const size_t rows = plan->schedule == PA_SCHEDULE_BALANCED
                            ? (size_t)decode_block_rows(args)
                            : (size_t)(args->batch > 0 ? args->batch : 0) * args->num_q_heads *
                                  args->q_len;
    *workspace_bytes = S > 1 ? rows * S * (args->head_dim + 1) * sizeof(float) : 0;
  }
  return PA_OK;
}

PA_EXPORT pa_status pa_decode(const pa_args *args, const pa_workspace *ws, void *stream) {
  pa_status st = check_sizes(args);
  if (st != PA_OK) return st;
  if (args->q_len > 8) return PA_ERR_INVALID_ARG;
  if (nothing_to_do(args)) return PA_OK;
  if ((st = check_pointers(args)) != PA_OK) return st;
  int32_t S, P;
  bool balanced;
  if ((st = check_workspace(args, ws, &S, &P, &balanced)) != PA_OK) return st;
  if (!balanced && (st = check_decode_grid(args, S)) != PA_OK) return st;
  const pa::LaunchParams p = make_params(args, S, P, balanced, ws);
  if ((st = enqueue_check(args, nullptr, (hipStream_t)stream)) != PA_OK) return st;
  return hip_status(pa::launch_decode(p, (pa::DType)args->dtype, (hipStream_t)stream));
}

PA_EXPORT pa_status pa_split_reduce(const pa_args *args, const pa_workspace *ws, void *stream) {
  pa_status st = check_sizes(args);
  if (st != PA_OK) return st;
  if (args->q_len > 8) return PA_ERR_INVALID_ARG;
  if (nothing_to_do(args)) return PA_OK;
  if ((st = check_pointers(args)) != PA_OK) return st;
  int32_t S, P;
  bool balanced;
  if ((st = check_workspace(args, ws, &S, &P, &balanced)) != PA_OK) return st;
  if (S == 1) return PA_OK;                  // pa_decode already wrote `out`
  if (balanced && ws->counters) return PA_OK;  // pa_decode merged the pieces itself
  const pa::LaunchParams p = make_params(args, S, P, balanced, ws);
  return hip_status(pa::launch_split_reduce(p, (pa::DType)args->dtype, (hipStream_t)stream));
}

namespace {

// Row tiles (128 packed rows) of one (request, kv head) of the bf16 prefill.
int64_t prefill_tiles(const pa_args *a) {
  return ((int64_t)(a->num_q_heads / a->num_kv_heads) * a->q_len + 127) / 128;
}

// Whether the bf16 prefill of `a` can run the key split.
bool prefill_splits(const pa_args *a) {
  return a->dtype == PA_DTYPE_BF16 && (int64_t)a->batch * prefill_tiles(a) <= pa::kSplitMaxPairs;
}

}  // namespace

PA_EXPORT pa_status pa_prefill_plan(const pa_args *args, int32_t num_cus, pa_workspace *plan,
                                    size_t *workspace_bytes) {
  pa_status st = check_sizes(args);
  if (st != PA_OK) return st;
  if (!plan) return PA_ERR_INVALID_ARG;
  plan->schedule = PA_SCHEDULE_KEY_SPLIT;
  plan->partition_tokens = 0;
  plan->num_splits = 0;
  plan->num_counters = 0;
  if (workspace_bytes) *workspace_bytes = 0;
  if (!prefill_splits(args)) return PA_OK;  // runs unsplit: no workspace
  // five piece slots per compute unit: the split sizes its pieces from the
  // slot count (at most 0.8 of the slots hold split pieces) and launches at
  // most half as many extra workgroups.  Measured against four: C5-like
  // prefill -5 to -11%, long prompts of 4096-16384 rows -3 to -5%, short
  // ones (2048 rows) +3%, chunked prefill within +-2%.
  const int cus = num_cus > 0 ? num_cus : 256;
  plan->num_splits = 5 * cus;
  plan->num_counters = plan->num_splits;
  if (workspace_bytes)
    *workspace_bytes = (size_t)plan->num_splits * (args->head_dim / 2 + 2) * 256 * sizeof(float);
  return PA_OK;
}

PA_EXPORT pa_status pa_prefill(const pa_args *args, const pa_workspace *ws, void *stream) {
  pa_status st = check_sizes(args);
  if (st != PA_OK) return st;
  if (nothing_to_do(args)) return PA_OK;
  if ((st = check_pointers(args)) != PA_OK) return st;
  const int32_t cap = args->max_pages * args->page_size;
  pa::LaunchParams p = make_params(args, 1, cap, false, nullptr);
  if (ws && ws->num_splits > 0) {
    // two slots at least: the pieces of split tiles take fewer than
    // 2 * floor(num_splits / 2) slots
    if (ws->schedule != PA_SCHEDULE_KEY_SPLIT || ws->num_splits < 2 || !ws->partial_out ||
        !ws->partial_lse ||
        !ws->counters || ws->num_counters < ws->num_splits || !aligned16(ws->partial_out) ||
        !aligned16(ws->partial_lse) || (reinterpret_cast<uintptr_t>(ws->counters) & 3u))
      return PA_ERR_WORKSPACE;
    if (prefill_splits(args)) {  // otherwise the call runs unsplit
      p.ws_o = ws->partial_out;
      p.ws_lse = ws->partial_lse;
      p.counters = ws->counters;
      p.num_splits = ws->num_splits;
    }
  }
  if (args->dtype == PA_DTYPE_BF16) {
    const int64_t tiles = prefill_tiles(args);
    if (tiles * args->num_kv_heads > INT32_MAX) return PA_ERR_INVALID_ARG;
    if (tiles * args->num_kv_heads * args->batch + ws_slots(p) > INT32_MAX) return PA_ERR_INVALID_ARG;
    if ((st = enqueue_check(args, nullptr, (hipStream_t)stream)) != PA_OK) return st;
    return hip_status(pa::launch_prefill_mfma(p, (hipStream_t)stream));
  }
  if ((st = check_decode_grid(args, 1)) != PA_OK) return st;
  if ((st = enqueue_check(args, nullptr, (hipStream_t)stream)) != PA_OK) return st;
  return hip_status(pa::launch_decode(p, (pa::DType)args->dtype, (hipStream_t)stream));
}

namespace {

// pa_attention's route: decode when the query rows of one kv head fit one
// decode row block (each K/V byte is then read once per kv head), else
// prefill (K/V read once per 128-row tile); a packed ragged call with more
// than one row bound routes each request (when some request can take the
// decode path at all).
int attention_route(const pa_args *a) {
  const int64_t G = a->num_q_heads / a->num_kv_heads;
  if (G * a->q_len <= 8) return PA_ROUTE_DECODE;
  if (a->query_start_loc && G <= 8) return PA_ROUTE_RAGGED;
  return PA_ROUTE_PREFILL;
}

// The decode part of a ragged call: the same call with one query row per
// request (its requests have at most one).
pa_args ragged_decode_args(const pa_args *a) {
  pa_args d = *a;
  d.q_len = 1;
  d.num_tokens = 0;  // sizes prefill grids only
  return d;
}

size_t round16(size_t x) { return (x + 15) / 16 * 16; }

// Plans of both parts of a ragged call.
pa_status ragged_plans(const pa_args *a, int32_t num_cus, pa_workspace *dec, pa_workspace *pre,
                       size_t *dec_bytes, size_t *pre_bytes) {
  const pa_args d = ragged_decode_args(a);
  memset(dec, 0, sizeof *dec);
  memset(pre, 0, sizeof *pre);
  pa_status st = pa_decode_plan(&d, num_cus, dec, dec_bytes);
  if (st != PA_OK) return st;
  if (dec->schedule != PA_SCHEDULE_BALANCED) return PA_ERR_UNSUPPORTED;  // batch above 2048
  return pa_prefill_plan(a, num_cus, pre, pre_bytes);
}

}  // namespace

PA_EXPORT pa_status pa_attention_plan(const pa_args *args, int32_t num_cus, pa_workspace *plan,
                                      size_t *workspace_bytes, int32_t *route) {
  pa_status st = check_sizes(args);
  if (st != PA_OK) return st;
  if (!plan) return PA_ERR_INVALID_ARG;
  const int r = attention_route(args);
  if (route) *route = r;
  plan->prefill_splits = 0;
  if (r == PA_ROUTE_DECODE) return pa_decode_plan(args, num_cus, plan, workspace_bytes);
  if (r == PA_ROUTE_PREFILL) return pa_prefill_plan(args, num_cus, plan, workspace_bytes);
  pa_workspace dec, pre;
  size_t db = 0, pb = 0;
  if ((st = ragged_plans(args, num_cus, &dec, &pre, &db, &pb)) != PA_OK) return st;
  const pa_args d = ragged_decode_args(args);
  const size_t rows = (size_t)decode_block_rows(&d);
  plan->schedule = PA_SCHEDULE_BALANCED;
  plan->partition_tokens = 0;
  plan->num_splits = dec.num_splits;
  plan->num_counters = dec.num_counters + pre.num_counters;
  plan->prefill_splits = pre.num_splits;
  if (workspace_bytes)
    *workspace_bytes = ((size_t)dec.num_splits * rows * args->head_dim +
                        round16((size_t)dec.num_splits * rows)) * sizeof(float) + pb;
  return PA_OK;
}

PA_EXPORT pa_status pa_attention(const pa_args *args, const pa_workspace *ws, void *stream) {
  pa_status st = check_sizes(args);
  if (st != PA_OK) return st;
  const int r = attention_route(args);
  if (r == PA_ROUTE_PREFILL) return pa_prefill(args, ws, stream);
  if (r == PA_ROUTE_DECODE) {
    if ((st = pa_decode(args, ws, stream)) != PA_OK) return st;
    const bool merged = ws && ws->schedule == PA_SCHEDULE_BALANCED && ws->counters;
    if (ws && ws->num_splits > 1 && !merged) return pa_split_reduce(args, ws, stream);
    return PA_OK;
  }
  // ragged: the decode part (requests of one row, merge fused) and the
  // prefill part (the others), one launch each, on `stream`
  if (nothing_to_do(args)) return PA_OK;
  if ((st = check_pointers(args)) != PA_OK) return st;
  pa_workspace dec, pre;
  size_t db = 0, pb = 0;
  if ((st = ragged_plans(args, 0, &dec, &pre, &db, &pb)) != PA_OK) return st;
  const pa_args d = ragged_decode_args(args);
  const size_t rows = (size_t)decode_block_rows(&d);
  const int64_t dec_counters = (int64_t)args->batch * decode_units(&d);
  if (!ws || ws->schedule != PA_SCHEDULE_BALANCED || !ws->partial_out || !ws->partial_lse ||
      !ws->counters || !aligned16(ws->partial_out) || !aligned16(ws->partial_lse) ||
      (reinterpret_cast<uintptr_t>(ws->counters) & 3u) ||
      (int64_t)ws->num_splits < dec_counters + 1 || ws->prefill_splits < 0 ||
      (int64_t)ws->num_counters < dec_counters)
    return PA_ERR_WORKSPACE;
  pa_workspace wd;
  memset(&wd, 0, sizeof wd);
  wd.partial_out = ws->partial_out;
  wd.partial_lse = ws->partial_lse;
  wd.num_splits = ws->num_splits;
  wd.schedule = PA_SCHEDULE_BALANCED;
  wd.num_counters = (int32_t)dec_counters;
  wd.counters = ws->counters;
  int32_t S, P;
  bool balanced;
  if ((st = check_workspace(&d, &wd, &S, &P, &balanced)) != PA_OK) return st;
  pa::LaunchParams pd = make_params(&d, S, P, balanced, &wd);
  pd.route = 1;
  if (args->dtype == PA_DTYPE_BF16) {
    const int64_t tiles = prefill_tiles(args);
    if (tiles * args->num_kv_heads * args->batch + ws->prefill_splits > INT32_MAX)
      return PA_ERR_INVALID_ARG;
  } else if ((st = check_decode_grid(args, 1)) != PA_OK) {
    return st;
  }
  // one check of the whole call (its metadata is the decode part's too)
  if ((st = enqueue_check(args, nullptr, (hipStream_t)stream)) != PA_OK) return st;
  hipError_t e = pa::launch_decode(pd, (pa::DType)args->dtype, (hipStream_t)stream);
  if (e != hipSuccess) return PA_ERR_HIP;
  // the prefill part, with the key split in the workspace's second region
  const int32_t cap = args->max_pages * args->page_size;
  pa::LaunchParams pp = make_params(args, 1, cap, false, nullptr);
  pp.route = 2;
  if (ws->prefill_splits >= 2 && prefill_splits(args)) {
    pp.ws_o = ws->partial_out + (size_t)ws->num_splits * rows * args->head_dim;
    pp.ws_lse = ws->partial_lse + round16((size_t)ws->num_splits * rows);
    pp.counters = ws->counters + dec_counters;
    pp.num_splits = ws->prefill_splits;
  }
  if (args->dtype == PA_DTYPE_BF16) {
    const int64_t tiles = prefill_tiles(args);
    if (tiles * args->num_kv_heads * args->batch + ws_slots(pp) > INT32_MAX)
      return PA_ERR_INVALID_ARG;
    return hip_status(pa::launch_prefill_mfma(pp, (hipStream_t)stream));
  }
  if ((st = check_decode_grid(args, 1)) != PA_OK) return st;
  return hip_status(pa::launch_decode(pp, (pa::DType)args->dtype, (hipStream_t)stream));
}

// ------------------------------------------------------------ shared prefixes
namespace {

// The prefix launch of a shared-prefix decode as prefill arguments: one
// request per group of max_group_size * q_len rows over the group's prefix
// keys, no mask (the kernels take the rows, keys and table from the groups).
pa_args prefix_launch_args(const pa_args *a, const pa_prefix_groups *g) {
  pa_args v = *a;
  v.batch = g->num_groups;
  v.q_len = g->max_group_size * a->q_len;
  v.query_lens = nullptr;
  v.query_start_loc = nullptr;
  v.num_tokens = 0;
  v.mask = PA_MASK_NONE;
  return v;
}

// Host-side checks of the groups (their contents are device data).
pa_status check_groups(const pa_args *a, const pa_prefix_groups *g) {
  if (!g) return PA_ERR_INVALID_ARG;
  if (a->dtype != PA_DTYPE_BF16) return PA_ERR_UNSUPPORTED;
  if (a->debug_trace || a->debug_visits) return PA_ERR_UNSUPPORTED;
  if (a->batch == 0) return PA_OK;
  if (g->num_groups < 0 || g->num_groups > a->batch || g->max_group_size < 1 ||
      g->max_group_size > a->batch)
    return PA_ERR_INVALID_ARG;
  if (!g->group_start || (g->num_groups > 0 && !g->prefix_lens) ||
      (reinterpret_cast<uintptr_t>(g->group_start) & 3u) ||
      (reinterpret_cast<uintptr_t>(g->prefix_lens) & 3u))
    return PA_ERR_INVALID_ARG;
  return PA_OK;
}

// Rows of the prefix states: every row of the call (an upper bound for
// packed rows).
size_t state_rows(const pa_args *a) {
  return (size_t)a->batch * a->num_q_heads * a->q_len;
}

}  // namespace

PA_EXPORT pa_status pa_decode_shared_plan(const pa_args *args, const pa_prefix_groups *groups,
                                          int32_t num_cus, pa_workspace *plan,
                                          size_t *workspace_bytes) {
  pa_status st = check_sizes(args);
  if (st != PA_OK) return st;
  if (!plan) return PA_ERR_INVALID_ARG;
  if (args->q_len > 8) return PA_ERR_INVALID_ARG;
  if ((st = check_groups(args, groups)) != PA_OK) return st;
  pa_workspace dec, pre;
  memset(&dec, 0, sizeof dec);
  memset(&pre, 0, sizeof pre);
  size_t db = 0, pb = 0;
  if ((st = pa_decode_plan(args, num_cus, &dec, &db)) != PA_OK) return st;
  if (dec.schedule != PA_SCHEDULE_BALANCED) return PA_ERR_UNSUPPORTED;  // batch above 2048
  if (args->batch > 0 && groups->num_groups > 0) {
    const pa_args v = prefix_launch_args(args, groups);
    if ((st = pa_prefill_plan(&v, num_cus, &pre, &pb)) != PA_OK) return st;
  }
  (void)pb;  // the prefix launch plans pieces but merges none: no split workspace
  const size_t R = (size_t)decode_block_rows(args);
  const size_t rows = state_rows(args);
  plan->schedule = PA_SCHEDULE_BALANCED;
  plan->partition_tokens = 0;
  plan->num_splits = dec.num_splits;
  plan->num_counters = dec.num_counters;
  plan->prefill_splits = pre.num_splits;
  if (workspace_bytes)
    *workspace_bytes = ((size_t)dec.num_splits * R * args->head_dim +
                        round16((size_t)dec.num_splits * R) +
                        rows * pa::kPrefixPieces * args->head_dim +
                        round16(rows * pa::kPrefixPieces) + round16(rows)) * sizeof(float);
  return PA_OK;
}

PA_EXPORT pa_status pa_decode_shared(const pa_args *args, const pa_prefix_groups *groups,
                                     const pa_workspace *ws, void *stream) {
  pa_status st = check_sizes(args);
  if (st != PA_OK) return st;
  if (args->q_len > 8) return PA_ERR_INVALID_ARG;
  if ((st = check_groups(args, groups)) != PA_OK) return st;
  if (nothing_to_do(args)) return PA_OK;
  if ((st = check_pointers(args)) != PA_OK) return st;
  const size_t R = (size_t)decode_block_rows(args);
  const int64_t dec_counters = (int64_t)args->batch * decode_units(args);
  if (!ws || ws->schedule != PA_SCHEDULE_BALANCED || !ws->partial_out || !ws->partial_lse ||
      !ws->counters || !aligned16(ws->partial_out) || !aligned16(ws->partial_lse) ||
      (reinterpret_cast<uintptr_t>(ws->counters) & 3u) ||
      (int64_t)ws->num_splits < dec_counters + 1 || ws->prefill_splits < 0 ||
      (int64_t)ws->num_counters < dec_counters)
    return PA_ERR_WORKSPACE;
  pa_workspace wd;
  memset(&wd, 0, sizeof wd);
  wd.partial_out = ws->partial_out;
  wd.partial_lse = ws->partial_lse;
  wd.num_splits = ws->num_splits;
  wd.schedule = PA_SCHEDULE_BALANCED;
  wd.num_counters = (int32_t)dec_counters;
  wd.counters = ws->counters;
  int32_t S, P;
  bool balanced;
  if ((st = check_workspace(args, &wd, &S, &P, &balanced)) != PA_OK) return st;
  const size_t rows = state_rows(args);
  float *state_o = ws->partial_out + (size_t)S * R * args->head_dim;
  float *state_lse = ws->partial_lse + round16((size_t)S * R);
  int32_t *state_n = reinterpret_cast<int32_t *>(state_lse + round16(rows * pa::kPrefixPieces));
  // the prefix launch: each group's member rows over its shared pages
  if (groups->num_groups > 0) {
    const pa_args v = prefix_launch_args(args, groups);
    const int32_t cap = args->max_pages * args->page_size;
    pa::LaunchParams pp = make_params(&v, 1, cap, false, nullptr);
    pp.grp_start = groups->group_start;
    pp.grp_pre = groups->prefix_lens;
    pp.num_groups = groups->num_groups;
    pp.prefix_pass = 1;
    pp.Lm = args->q_len;
    pp.qsl = args->query_start_loc;  // member rows are addressed as in the call
    pp.num_tokens = 0;
    pp.ql = args->query_lens;
    pp.pre_o = state_o;
    pp.pre_lse = state_lse;
    pp.pre_n = state_n;
    // the key split plans with prefill_splits slots; its pieces leave row
    // states and merge nothing, so they need no split workspace
    if (ws->prefill_splits >= 2 && prefill_splits(&v)) pp.num_splits = ws->prefill_splits;
    const int64_t tiles = prefill_tiles(&v);
    if (tiles * v.num_kv_heads * v.batch + pp.num_splits / 2 + 1 > INT32_MAX)
      return PA_ERR_INVALID_ARG;
    if ((st = enqueue_check(args, groups, (hipStream_t)stream)) != PA_OK) return st;
    if (pa::launch_prefill_mfma(pp, (hipStream_t)stream) != hipSuccess) return PA_ERR_HIP;
  } else if ((st = enqueue_check(args, groups, (hipStream_t)stream)) != PA_OK) {
    return st;
  }
  // the decode launch: keys past each request's prefix, merged with its state
  pa::LaunchParams pd = make_params(args, S, P, balanced, &wd);
  pd.grp_start = groups->group_start;
  pd.grp_pre = groups->prefix_lens;
  pd.num_groups = groups->num_groups;
  pd.pre_o = state_o;
  pd.pre_lse = state_lse;
  pd.pre_n = state_n;
  return hip_status(pa::launch_decode(pd, (pa::DType)args->dtype, (hipStream_t)stream));
}

PA_EXPORT pa_status pa_append(const pa_append_args *args, void *stream) {
  if (!args) return PA_ERR_INVALID_ARG;
  const pa_append_args *a = args;
  if (a->num_tokens < 0 || a->num_kv_heads < 1 || a->head_dim < 1 || a->num_pages < 1 ||
      a->page_size < 1)
    return PA_ERR_INVALID_ARG;
  if ((int64_t)a->num_pages * a->page_size > INT32_MAX) return PA_ERR_INVALID_ARG;
  if (a->dtype != PA_DTYPE_F32 && a->dtype != PA_DTYPE_BF16) return PA_ERR_UNSUPPORTED;
  if (a->head_dim != 64 && a->head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (a->cache_dtype != PA_KV_SAME && a->cache_dtype != PA_KV_FP8_E4M3) return PA_ERR_INVALID_ARG;
  const bool fp8 = a->cache_dtype == PA_KV_FP8_E4M3;
  if (fp8) {
    if (!(a->k_scale > 0.f) || !isfinite(a->k_scale) || !(a->v_scale > 0.f) ||
        !isfinite(a->v_scale))
      return PA_ERR_INVALID_ARG;
    if (a->dtype != PA_DTYPE_BF16) return PA_ERR_UNSUPPORTED;
  }
  if (!a->key_pages || !a->value_pages || !aligned16(a->key_pages) ||
      !aligned16(a->value_pages))
    return PA_ERR_INVALID_ARG;
  if (a->num_tokens == 0) return PA_OK;
  if (!a->key || !a->value || !a->slot_mapping || !aligned16(a->key) || !aligned16(a->value))
    return PA_ERR_INVALID_ARG;
  pa::AppendParams p{};
  p.k = a->key;
  p.v = a->value;
  p.slots = a->slot_mapping;
  p.kp = a->key_pages;
  p.vp = a->value_pages;
  p.tokens = a->num_tokens;
  p.Hkv = a->num_kv_heads;
  p.ps = a->page_size;
  p.num_slots = a->num_pages * a->page_size;
  p.row_bytes = a->head_dim * (a->dtype == PA_DTYPE_F32 ? 4 : 2);
  p.fp8 = fp8 ? 1 : 0;
  p.k_scale = fp8 ? a->k_scale : 1.f;
  p.v_scale = fp8 ? a->v_scale : 1.f;
  return hip_status(pa::launch_append(p, (hipStream_t)stream));
}

// ------------------------------------------------------------- no allocation
// pa_decode_noalloc: pa_decode with the balanced schedule and the fused
// merge, whose partial states and arrival counters live in a library-owned
// device array instead of a caller workspace.  Layout of `scratch`: the
// arrival counters (kScratchCounters uint32), then the pieces' log-sum-exps
// (S x R fp32), then their partial outputs (S x R x D fp32), each region
// starting on a 256-byte boundary.
namespace {

constexpr size_t kScratchBytes = size_t(32) << 20;  // 32 MiB per device
constexpr int64_t kScratchCounters = int64_t(1) << 16;
constexpr size_t kScratchCounterBytes = size_t(kScratchCounters) * 4;

// In host code `scratch` names a host-side stand-in, not device memory: the
// device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

__global__ void zero_u32(uint32_t *p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch[kMaxDevices] = {nullptr};

size_t round256(size_t x) { return (x + 255) & ~size_t(255); }

// The current device's copy of `scratch`.  The first call on a device looks
// its address up (that device current) and enqueues a fill kernel that
// clears the counters on `stream` (kernels leave them zero after every
// call, so one clearing is enough; a fill kernel rather than a memset keeps
// the call capturable).
pa_status scratch_of_device(hipStream_t stream, unsigned char **base) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return PA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return PA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return PA_ERR_HIP;
    hipLaunchKernelGGL(zero_u32, dim3(64), dim3(256), 0, stream, static_cast<uint32_t *>(p),
                       kScratchCounters);
    if (hipGetLastError() != hipSuccess) return PA_ERR_HIP;
    g_scratch[dev] = p;
  }
  *base = static_cast<unsigned char *>(g_scratch[dev]);
  return PA_OK;
}

}  // namespace

PA_EXPORT pa_status pa_decode_noalloc(const pa_args *args, void *stream) {
  pa_status st = check_sizes(args);
  if (st != PA_OK) return st;
  if (args->q_len > 8) return PA_ERR_INVALID_ARG;
  if (nothing_to_do(args)) return PA_OK;
  if ((st = check_pointers(args)) != PA_OK) return st;
  pa_workspace ws;
  memset(&ws, 0, sizeof ws);
  size_t state_bytes = 0;
  if ((st = pa_decode_plan(args, 0, &ws, &state_bytes)) != PA_OK) return st;
  // the balanced schedule with its fused merge is the only plan the scratch
  // serves; its size must fit
  if (ws.schedule != PA_SCHEDULE_BALANCED) return PA_ERR_SCRATCH;
  const size_t rows = (size_t)decode_block_rows(args);
  const size_t lse_bytes = round256((size_t)ws.num_splits * rows * sizeof(float));
  const size_t out_bytes = (size_t)ws.num_splits * rows * args->head_dim * sizeof(float);
  if ((int64_t)ws.num_counters > kScratchCounters ||
      kScratchCounterBytes + lse_bytes + out_bytes > kScratchBytes)
    return PA_ERR_SCRATCH;
  (void)state_bytes;
  unsigned char *base = nullptr;
  if ((st = scratch_of_device((hipStream_t)stream, &base)) != PA_OK) return st;
  ws.counters = reinterpret_cast<uint32_t *>(base);
  ws.partial_lse = reinterpret_cast<float *>(base + kScratchCounterBytes);
  ws.partial_out = reinterpret_cast<float *>(base + kScratchCounterBytes + lse_bytes);
  return pa_decode(args, &ws, stream);
}
