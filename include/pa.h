/*
 * pa.h -- C ABI of the paged-attention read path for AMD Instinct MI355X
 * (gfx950).  libpa.so implements it with hand-written HIP kernels.
 *
 * The operation is the paged_attention contract of tiny-llm "Week 3 Day 4:
 * Direct Paged Attention" (section "The Paged Attention API"): every query row
 * attends over the keys/values of its request, which live in a shared page
 * pool.  Logical key j of request b is found by translating it through the
 * block table -- logical page j / page_size, physical page
 * block_table[b][j / page_size], slot j % page_size (sections "Why
 * block_table Matters" and "How This Maps to tiny-llm") -- and only the first
 * context_lens[b] keys are visible.  Tiles of K/V are folded into the output
 * with the online-softmax recurrence of the same page's "Task 2" (running max,
 * rescaled running sum and output, one division at the end); no dense K/V
 * tensor is ever built.  The metadata set matches PagedKvMetadata of anllm
 * "Tutorial 13" (section 6).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All data pointers are DEVICE pointers owned by the caller; the library
 *    never allocates, frees or synchronises.  Work is enqueued on `stream`
 *    (a hipStream_t; NULL means the null stream) and the call returns at once.
 *    A call enqueues kernel launches only (no memset or copy), and every
 *    kernel leaves the workspace's arrival counters at zero, so calls can be
 *    captured into a HIP graph and replayed (plan and workspace set up
 *    before the capture).
 *  - Layouts are dense row-major with no padding:
 *      query, out        [B, H_q, L, D]
 *      key/value_pages   [num_pages, H_kv, page_size, D]
 *      block_table       [B, max_pages] int32; entries at or after logical
 *                        page ceil(context_lens[b] / page_size) are never read
 *                        (pad them with -1)
 *      context_lens      [B] int32: visible keys of request b, including the
 *                        K/V of its own new query rows
 *      query_lens        [B] int32 or NULL (= L for every request): valid
 *                        query rows of request b; rows i >= query_lens[b] are
 *                        written as zeros
 *  - dtype applies to query, the pages and out alike: PA_DTYPE_F32 or
 *    PA_DTYPE_BF16 (bfloat16 bits).  Scores, softmax statistics and the
 *    accumulator are fp32; a bf16 output is rounded to nearest-even once.
 *  - head_dim must be 64 or 128.  Query head h reads kv head h / (H_q / H_kv).
 *  - Causal rows are bottom-right aligned: row i of request b is position
 *    context_lens[b] - query_lens[b] + i and sees keys j <= that position.
 *    With L = 1 the two masks coincide.
 *  - A row with no visible key (context 0) is written as zeros.
 *  - query, the pages, out and the workspace must be 16-byte aligned.
 *
 * Errors: arguments are validated synchronously before anything is enqueued.
 * A rejected call enqueues nothing and returns a negative pa_status.  The
 * device-side contract (block-table entries that must be read lie in
 * [0, num_pages); context_lens[b] <= max_pages * page_size; 0 <= query_lens[b]
 * <= L; with a causal mask query_lens[b] <= context_lens[b]) is taken on trust
 * and violating it is undefined behaviour.  Kernel faults surface at the
 * caller's next synchronisation.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_ABI_VERSION 12

typedef enum {
  PA_OK = 0,
  PA_ERR_INVALID_ARG = -1,  /* null pointer, bad size, bad scale/mask, misalignment */
  PA_ERR_UNSUPPORTED = -2,  /* head_dim or dtype outside what the kernels implement */
  PA_ERR_WORKSPACE = -3,    /* split workspace missing, too small or inconsistent */
  PA_ERR_HIP = -4,          /* the HIP runtime refused a launch */
  PA_ERR_SCRATCH = -5       /* pa_decode_noalloc: the call needs more than the
                               library scratch holds */
} pa_status;

typedef enum { PA_DTYPE_F32 = 0, PA_DTYPE_BF16 = 1 } pa_dtype;
typedef enum { PA_MASK_NONE = 0, PA_MASK_CAUSAL = 1 } pa_mask;

/* Element type of the K/V pages ("Reading vLLM's PagedAttention Kernel",
 * section 3.2: the cache write takes a kv-cache dtype and per-tensor k/v
 * scales).  PA_KV_SAME: the pages hold `dtype` elements.  PA_KV_FP8_E4M3:
 * the pages hold one byte per element, an 8-bit float in the OCP E4M3
 * encoding (bit 7 sign, bits 6..3 exponent with bias 7, bits 2..0
 * mantissa; exponent 0 subnormal; s.1111.111 NaN; no infinity), and an
 * element's value is its code's value times k_scale (keys) or v_scale
 * (values). */
typedef enum { PA_KV_SAME = 0, PA_KV_FP8_E4M3 = 1 } pa_kv_dtype;

/* Flags of the contract check (pa_args.debug_errors).  The kernels take the
 * metadata on trust (tiny-llm "Week 3 Day 4", "What Must Hold, and What
 * Breaks If It Doesn't": a page id outside the pool, or a context longer
 * than its block-table row, reads memory that is not the request's). */
typedef enum {
  PA_DEBUG_BAD_PAGE = 1,    /* a block-table entry the call reads is outside [0, num_pages) */
  PA_DEBUG_BAD_CONTEXT = 2, /* a context length < 0 or > max_pages * page_size */
  PA_DEBUG_BAD_ROWS = 4,    /* query rows outside [0, q_len] (query_lens, or
                               query_start_loc not 0 .. nondecreasing), or a
                               causal request with keys but fewer keys than rows */
  PA_DEBUG_BAD_GROUPS = 8   /* pa_decode_shared: groups or prefix lengths outside
                               their contract, or a member's table that differs
                               from its group's first member on the shared pages */
} pa_debug_flag;

typedef struct pa_args {
  const void *query;           /* [B, H_q, L, D] */
  const void *key_pages;       /* [num_pages, H_kv, page_size, D] */
  const void *value_pages;     /* [num_pages, H_kv, page_size, D] */
  const int32_t *block_table;  /* [B, max_pages] */
  const int32_t *context_lens; /* [B] */
  const int32_t *query_lens;   /* [B] or NULL */
  void *out;                   /* [B, H_q, L, D] */
  int32_t batch;               /* B >= 0 (0: nothing to do) */
  int32_t num_q_heads;         /* H_q, a multiple of H_kv */
  int32_t num_kv_heads;        /* H_kv >= 1 */
  int32_t q_len;               /* L >= 1 */
  int32_t head_dim;            /* D in {64, 128} */
  int32_t num_pages;           /* pool size >= 1 */
  int32_t page_size;           /* tokens per page >= 1 */
  int32_t max_pages;           /* block-table row length >= 1 */
  int32_t dtype;               /* pa_dtype */
  int32_t mask;                /* pa_mask */
  float scale;                 /* score scale, finite and > 0 (1/sqrt(D) is usual) */
  /* Debug outputs (NULL in normal use; either one selects the instrumented
   * kernels: the same staging and load code as the production kernels of
   * the call, plus the records).  debug_trace [B, max_pages*page_size, 2]
   * int32 receives, for every logical key the kernels read, the (physical
   * page, slot) decoded from the address that the load of the key actually
   * used; other entries are left as the caller set them.  debug_visits [B,
   * H_kv, max_pages*page_size] int32 is incremented once per key each time
   * a work item loads it for folding into the softmax state, under the kv
   * head that the load address points at; only the work items whose rows
   * include the last valid query row of the request count, so a correct
   * walk leaves exactly 1 for j < context_lens[b] and 0 beyond.  The caller
   * zeroes debug_visits. */
  int32_t *debug_trace;
  int32_t *debug_visits;
  /* Page element type (pa_kv_dtype; 0 = PA_KV_SAME).  PA_KV_FP8_E4M3 needs
   * dtype PA_DTYPE_BF16 (query and out) and head_dim 128; every read entry
   * point takes it. */
  int32_t kv_dtype;
  float k_scale;               /* fp8 pages: finite and > 0 (ignored otherwise) */
  float v_scale;               /* fp8 pages: finite and > 0 (ignored otherwise) */
  /* Packed (ragged) query rows, or NULL.  When given, query and out are
   * [T, H_q, D] with T = query_start_loc[batch]: request b owns rows
   * query_start_loc[b] .. query_start_loc[b + 1] - 1 (0 = query_start_loc[0]
   * <= ... nondecreasing), and no padding rows exist or are written.
   * q_len is then an upper bound on every request's row count (it sizes
   * tiles and plans), and query_lens must be NULL.  A call with no row at
   * all (T = 0) passes NULL query and out and does nothing. */
  const int32_t *query_start_loc;
  /* Packed rows only: T = query_start_loc[batch] (the rows of query and
   * out), or 0 if the caller does not give it; 0 <= num_tokens <= batch *
   * q_len.  It only sizes the prefill grid (a ragged call of many one-row
   * requests then launches no workgroups for their tiles); the kernels
   * read the row counts from query_start_loc.  Taken on trust: a value
   * below the true T leaves rows unwritten. */
  int32_t num_tokens;
  /* Contract check (debug mode), or NULL.  When given: int32 [2] in device
   * memory, which the caller zeroes.  Before its kernels, the call enqueues
   * a check that reads only the metadata (every block-table entry j <
   * ceil(min(context_lens[b], max_pages * page_size) / page_size) of every
   * request, the context lengths, the query rows, and the groups of
   * pa_decode_shared), ORs pa_debug_flag bits into debug_errors[0] and adds
   * the number of out-of-pool entries to debug_errors[1].  Every kernel of
   * the call reads debug_errors[0] first and, when it is nonzero, returns
   * without reading K/V or writing any output, workspace or counter; the
   * caller reads the word after synchronising.  Without it, a broken
   * contract is undefined behaviour (a page id outside the pool reads
   * outside the pool).  pa_append does not take it (its slots are checked
   * in every call); pa_split_reduce reads it and checks nothing itself. */
  int32_t *debug_errors;
} pa_args;

/* How pa_decode divides a call's keys among the waves of the GPU. */
typedef enum pa_schedule {
  /* Fixed partitions ("Reading vLLM's PagedAttention Kernel", section 3.3:
   * a long context is cut into partitions computed in parallel and combined
   * afterwards).  Partition s covers keys
   * [s * partition_tokens, min((s + 1) * partition_tokens, context_len)) of
   * every (request, kv head, row block); one wave walks each.  num_splits ==
   * 1 is the single-pass decode (no workspace needed). */
  PA_SCHEDULE_PARTITIONS = 0,
  /* Equal work per wave: the keys of every (request, kv head, row block),
   * in steps of STEP keys (16 for bf16 with head_dim 128; 4096 / (head_dim *
   * element bytes) in general), each row block preceded by a few setup
   * positions that stand for the cost of starting it, are laid out
   * request-major and cut into one contiguous run per wave of a grid that
   * fills the GPU, so ragged context lengths cost no idle waves.  A row block is R query rows of one kv head
   * (R = 1, 2, 4 or 8: the smallest that holds G * L, at most 8), and a
   * request has U = H_kv * ceil(G * L / R) of them.  Row block r of the call
   * (r = b * U + u) walked in part by wave w leaves its partial state in
   * piece slot r + w; one walked by a single wave is written to `out`
   * directly.  num_splits is the number of piece slots: at least B * U + 1
   * (the library uses at most num_splits - B * U waves), and batch <= 2048.
   * With `counters` (B * U of them) the merge is fused into pa_decode: the
   * last wave to finish a row block's piece merges its pieces, and
   * pa_split_reduce has nothing left to do. */
  PA_SCHEDULE_BALANCED = 1,
  PA_SCHEDULE_KEY_SPLIT = 2  /* bf16 prefill: key ranges split and merged */
} pa_schedule;

/* Split-KV workspace of the decode path: normalised partial outputs and the
 * natural-log log-sum-exp of their scaled scores (-inf: no visible key),
 *   partitions:  partial_out fp32 [B, H_q, L, num_splits, D],
 *                partial_lse fp32 [B, H_q, L, num_splits];
 *   balanced:    partial_out fp32 [num_splits, R, D],
 *                partial_lse fp32 [num_splits, R].
 * Both are caller-owned device memory of the size pa_decode_plan reports;
 * pa_decode overwrites them and pa_split_reduce reads them, so calls that
 * share one workspace must not overlap in time (same stream, or
 * synchronised).  With schedule == PA_SCHEDULE_PARTITIONS and num_splits ==
 * 1 the buffers may be NULL and pa_decode writes `out`. */
typedef struct pa_workspace {
  float *partial_out;
  float *partial_lse;
  int32_t num_splits;        /* partitions (>= 1), or piece slots (balanced) */
  int32_t partition_tokens;  /* partitions: > 0, a multiple of page_size; balanced: ignored */
  int32_t schedule;          /* pa_schedule */
  int32_t num_counters;      /* balanced: B * U (set by pa_decode_plan); partitions: 0 */
  /* Balanced only, optional: uint32 [num_counters] counters in device
   * memory (one arrival counter per row block).  The
   * caller zeroes them once before first use; every call leaves them zero.
   * NULL: pa_decode leaves the pieces' states and pa_split_reduce merges. */
  uint32_t *counters;
  /* Ragged route of pa_attention only: the key-split slots of its prefill
   * part (0 otherwise). */
  int32_t prefill_splits;
} pa_workspace;

/* Choose the plan of pa_decode for `args` (only the sizes in `args` are
 * read; no pointer is dereferenced and nothing runs on the GPU).
 * On input plan->partition_tokens > 0 requests the partition schedule with
 * that partition size (rounded up to a multiple of page_size); 0 lets the
 * library choose: the balanced schedule when batch <= 2048, sized for
 * `num_cus` compute units (0: 256, the MI355X count), else partitions
 * chosen from the maximum context max_pages * page_size.
 * On return plan->schedule, num_splits, partition_tokens and num_counters
 * are set, the buffer pointers are left untouched, and *workspace_bytes (if
 * not NULL) is the total size of partial_out plus partial_lse (0 when no
 * split); the counters take num_counters * 4 bytes more. */
pa_status pa_decode_plan(const pa_args *args, int32_t num_cus, pa_workspace *plan,
                         size_t *workspace_bytes);

/* Decode: query rows L <= 8 (one-token decode and short chunks).  A wave
 * walks the pages of one (request, kv head, row block) at a time with the
 * G * L query rows of that kv head held in registers, so every K/V byte is
 * read once per row block.  A single-pass plan writes `out`; otherwise
 * pa_split_reduce must follow on the same stream. */
pa_status pa_decode(const pa_args *args, const pa_workspace *ws, void *stream);

/* Log-sum-exp merge of the partial states pa_decode left in `ws` into
 * `out`: M = max_s lse_s, out = sum_s exp(lse_s - M) o_s / sum_s exp(lse_s - M),
 * over the partitions s < ceil(context_lens[b] / partition_tokens), or over
 * the pieces of the balanced schedule; rows with no visible key get zeros.
 * `args` and `ws` must be those of that pa_decode. */
pa_status pa_split_reduce(const pa_args *args, const pa_workspace *ws, void *stream);

/* Plan of pa_prefill for `args` (sizes only; nothing runs on the GPU).
 * The bf16 prefill can split the key range of a row tile into pieces walked
 * by separate workgroups and merged with the log-sum-exp rule ("Reading
 * vLLM's PagedAttention Kernel", section 3.3: partial results combined
 * afterwards), so that one long context in a batch does not bound the call.
 * On return plan->schedule = PA_SCHEDULE_KEY_SPLIT and plan->num_splits =
 * num_counters = the slots of the split (5 per compute unit, `num_cus` 0:
 * 256), or 0 when the call cannot split (fp32, or batch * ceil(G * L / 128)
 * above 2048): no workspace then.  *workspace_bytes (if not NULL) is the size
 * of partial_out plus partial_lse; the counters take num_counters * 4 bytes
 * more. */
pa_status pa_prefill_plan(const pa_args *args, int32_t num_cus, pa_workspace *plan,
                          size_t *workspace_bytes);

/* Prefill: any L >= 1 (chunked prefill after a cached prefix).  bf16 runs on
 * the MFMA kernel (K/V tiles staged page by page through LDS, QK^T and PV on
 * bf16 matrix cores, fp32 statistics); fp32 runs on a vector-ALU kernel.
 * fp8 pages (bf16 query) run on the MFMA kernel too: the codes are loaded
 * into LDS as they are and widened exactly to bf16 by the operand reads
 * (pools of 2 GiB and more with a page size that is not a multiple of 8
 * widen them on their way into LDS), k_scale scales the scores and v_scale
 * the output.
 * `ws` is NULL (no split) or a workspace of pa_prefill_plan: partial_out
 * fp32 [num_splits, D / 8, 256, 4] and partial_lse fp32 [num_splits, 2, 256]
 * (the state of a piece: the accumulators, reference maxima and row sums of
 * the workgroup's 256 threads), counters uint32 [num_counters], zeroed by the
 * caller once and left zero by every call.  Calls sharing a workspace must
 * not overlap in time.  PA_ERR_WORKSPACE: a workspace that is inconsistent
 * (wrong schedule, fewer than 2 slots or counters than slots, missing
 * buffers or counters, misaligned). */
pa_status pa_prefill(const pa_args *args, const pa_workspace *ws, void *stream);

/* ------------------------------------------------------------------ router
 * One call for any query length: the shape decision sits at the boundary
 * (tiny-llm "Week 3 Day 4", "Choose a Schedule for Each Query Shape": one
 * tile shape cannot serve decode and prefill well, and the choice belongs in
 * the extension's dispatch).  The decode kernel holds the G * L query rows of
 * a kv head in one row block of at most 8 rows and reads every K/V byte once
 * per row block; the prefill kernel reads K/V once per 128-row tile.  So
 * pa_attention runs the decode path when G * L <= 8 (G = H_q / H_kv) and
 * the prefill path otherwise.  Measured on MI355X with 64 requests of
 * U[128, 4096] keys, H_q 32, H_kv 8, D 128, bf16: L = 1 decode 125 us vs
 * prefill 191 us; L = 2 149 vs 171; L = 4 298 vs 195; L = 8 627 vs 195. */
typedef enum { PA_ROUTE_DECODE = 0, PA_ROUTE_PREFILL = 1, PA_ROUTE_RAGGED = 2 } pa_route;

/* Ragged batches (packed rows, query_start_loc given, q_len > 1): the shape
 * decision is taken per request, in one call on one stream.  A request of
 * one query row (G <= 8) takes the decode path, every other request the
 * prefill path; pa_attention enqueues the decode kernel for the first kind
 * and the prefill kernel for the second, each skipping the other's
 * requests.  Route PA_ROUTE_RAGGED; its workspace holds both paths' parts,
 * each in its own region:
 *   partial_out  decode: num_splits * R * head_dim floats, then prefill:
 *                prefill_splits * head_dim * 128 floats;
 *   partial_lse  decode: num_splits * R floats rounded up to a multiple of
 *                16, then prefill: prefill_splits * 512 floats;
 *   counters     decode: batch * H_kv, then prefill: prefill_splits;
 * with R the decode rows per block (the smallest of 1, 2, 4, 8 that holds G),
 * num_splits the decode plan's piece slots (balanced schedule, merge fused)
 * and prefill_splits the prefill plan's key-split slots.  The counters are
 * zeroed once by the caller and left zero by every call. */

/* The plan of pa_attention: *route (if not NULL) receives the path, and
 * `plan` / *workspace_bytes are those of pa_decode_plan (decode route;
 * plan->partition_tokens on input as there), pa_prefill_plan, or for the
 * ragged route both (plan->num_splits, num_counters: the decode part;
 * plan->prefill_splits: the prefill part; *workspace_bytes: all of
 * partial_out and partial_lse). */
pa_status pa_attention_plan(const pa_args *args, int32_t num_cus, pa_workspace *plan,
                            size_t *workspace_bytes, int32_t *route);

/* Attention for any L >= 1 on the route of pa_attention_plan, with that
 * plan's workspace (or NULL where the route allows it): the decode route
 * runs pa_decode and, when its pieces are not merged in the kernel (a split
 * without arrival counters), pa_split_reduce; the prefill route runs
 * pa_prefill.  Errors as for those calls. */
pa_status pa_attention(const pa_args *args, const pa_workspace *ws, void *stream);

/* ------------------------------------------------------- shared prefixes
 * Block sharing across requests ("Reading vLLM's PagedAttention Kernel",
 * section 1 "Intuition" and section 2 "Mental model": two block tables may
 * name the same physical block, which is what prefix caching builds on).
 * When the requests of a group share their first pages, pa_decode_shared
 * reads those pages once for the whole group instead of once per request:
 * a prefix launch (the bf16 matrix-core kernel, one request per group whose
 * query rows are all the members' rows, no mask) leaves each member row's
 * state over the prefix -- normalised output and log-sum-exp -- and the
 * decode kernel walks each request's keys past the prefix and merges that
 * state into the row's other partial states with the log-sum-exp rule
 * (section 3.3).  The result is the same attention as pa_decode's, up to
 * rounding order.
 *
 * Groups are consecutive ranges of requests from the start of the batch:
 * group k holds requests group_start[k] .. group_start[k + 1] - 1
 * (group_start[0] = 0, nondecreasing, group_start[num_groups] <= batch), and
 * the requests from group_start[num_groups] on share nothing (a caller moves
 * the sharers of each prefix next to each other, at the front).  num_groups
 * 0 is a plain decode.  Group k shares its first
 * P_k = prefix_lens[k] - prefix_lens[k] % page_size keys (whole pages only;
 * a partial page is walked by each request).  Device-side contract, taken on
 * trust like the block-table contract: every member's block table names the
 * same physical pages as the group's first member for logical pages below
 * P_k / page_size, and every member b with query rows has P_k <=
 * context_lens[b] - (its query rows) (every row then sees the whole prefix);
 * group k has at most max_group_size requests. */
typedef struct pa_prefix_groups {
  const int32_t *group_start; /* [num_groups + 1] int32, device */
  const int32_t *prefix_lens; /* [num_groups] int32, device: shared keys of each group
                                 (may be NULL when num_groups is 0) */
  int32_t num_groups;         /* 0 .. batch */
  int32_t max_group_size;     /* >= 1: bound on the requests of a group */
} pa_prefix_groups;

/* Plan of pa_decode_shared (sizes only; nothing runs on the GPU): the decode
 * part's balanced plan with the merge fused (plan->num_splits piece slots,
 * plan->num_counters = batch * U counters) and the slot count the prefix
 * launch plans its key split with (plan->prefill_splits, 0: unsplit).  The
 * prefix launch cuts each row tile's prefix keys into at most 16 pieces and
 * every piece leaves its own state of each member row (no merge there: the
 * decode launch folds a row's prefix states into the row's merge).
 * Workspace layout, each part in its own region (N = batch * H_q * q_len
 * rows, states by output row index):
 *   partial_out  decode: num_splits * R * head_dim floats, then the prefix
 *                states: N * 16 * head_dim floats;
 *   partial_lse  decode: num_splits * R floats rounded up to a multiple of
 *                16, then N * 16 log-sum-exps rounded up to a multiple of
 *                16, then N int32 piece counts (rounded up to 16);
 *   counters     decode: batch * U;
 * R, U as for the balanced schedule.  *workspace_bytes is all of partial_out
 * and partial_lse.  PA_ERR_UNSUPPORTED: dtype other than bf16, debug
 * outputs, or a batch the balanced schedule does not take. */
pa_status pa_decode_shared_plan(const pa_args *args, const pa_prefix_groups *groups,
                                int32_t num_cus, pa_workspace *plan, size_t *workspace_bytes);

/* Decode (q_len <= 8, as pa_decode) with the shared prefixes of `groups`
 * read once per group: the prefix launch, then the decode launch, both on
 * `stream`, with the workspace of pa_decode_shared_plan (counters zeroed
 * once by the caller, left zero by every call).  Errors as for pa_decode;
 * PA_ERR_INVALID_ARG also for a NULL or misaligned group array or
 * num_groups / max_group_size out of range. */
pa_status pa_decode_shared(const pa_args *args, const pa_prefix_groups *groups,
                           const pa_workspace *ws, void *stream);

/* ---------------------------------------------------------------- write path
 * The K/V write that precedes attention on every step: each new token's key
 * and value rows are scattered to their physical slots in the page pool
 * ("Reading vLLM's PagedAttention Kernel", section 3.2: the write path maps
 * every token to a flat slot, physical page * page_size + offset in the page,
 * and the read path gathers the slots back through the block table).  The
 * runtime chooses the slots -- in tiny-llm "Week 3 Day 4" ("Decode Metadata")
 * and anllm "Tutorial 13" (section 4, the request cache's append) a request
 * fills its tail page before a new page is allocated -- and passes them in
 * slot_mapping.  Every element of every row is copied bit for bit; nothing
 * else in the pool is written.
 *
 * Layouts (dense, row-major, 16-byte aligned):
 *   key, value            [num_tokens, num_kv_heads, head_dim]   (dtype)
 *   slot_mapping          [num_tokens] int32; slot s of token t receives its
 *                         rows in page s / page_size at offset s % page_size
 *                         of every kv head; s < 0 (padding) or
 *                         s >= num_pages * page_size skips the token
 *   key_pages, value_pages [num_pages, num_kv_heads, page_size, head_dim]
 * Two tokens with the same slot race (which one lands is unspecified).
 * The pages may be read by attention calls enqueued after this one on the
 * same stream. */
typedef struct pa_append_args {
  const void *key;               /* [num_tokens, num_kv_heads, head_dim] */
  const void *value;             /* [num_tokens, num_kv_heads, head_dim] */
  const int32_t *slot_mapping;   /* [num_tokens] */
  void *key_pages;               /* [num_pages, num_kv_heads, page_size, head_dim] */
  void *value_pages;             /* [num_pages, num_kv_heads, page_size, head_dim] */
  int32_t num_tokens;            /* >= 0 (0: nothing to do) */
  int32_t num_kv_heads;          /* >= 1 */
  int32_t head_dim;              /* 64 or 128 */
  int32_t num_pages;             /* >= 1 */
  int32_t page_size;             /* >= 1 */
  int32_t dtype;                 /* pa_dtype of key and value (and of the pages when
                                    cache_dtype is PA_KV_SAME) */
  /* pa_kv_dtype of the pages (0 = PA_KV_SAME: rows copied bit for bit).
   * PA_KV_FP8_E4M3 (key/value bf16): each element x is stored as the E4M3
   * code nearest to x / scale, the division done in fp32 and correctly
   * rounded, ties to the code with an even mantissa, magnitudes beyond 448
   * saturated to 448, NaN kept NaN (k_scale for keys, v_scale for values,
   * both finite and > 0). */
  int32_t cache_dtype;
  float k_scale;
  float v_scale;
} pa_append_args;

/* Scatter the rows of `key` and `value` into the page pool (quantising
 * them for an fp8 pool).
 * PA_ERR_INVALID_ARG: a NULL or misaligned pointer, a size out of range, a
 * bad scale, or a pool of 2^31 slots or more; PA_ERR_UNSUPPORTED: head_dim,
 * dtype or cache_dtype. */
pa_status pa_append(const pa_append_args *args, void *stream);

/* -------------------------------------------------------- no allocation
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.
 *
 * pa_decode_noalloc is pa_decode with the plan pa_decode_plan chooses for
 * `args` (num_cus 0) -- which must be the balanced schedule -- and the merge
 * fused in the kernel, but its partial states and arrival counters live in
 * a library-owned device array of 32 MiB per device, held from the first
 * call on a device until the process ends.  It allocates nothing, calls no
 * hipMalloc/hipFree, and enqueues kernels only on `stream`: on the first
 * call on a device it looks the array up and enqueues a fill kernel that
 * clears the counters (every call leaves them zero afterwards); then the
 * decode kernel.  The caller passes inputs and outputs as for pa_decode.
 * Limits: at most 65536 row blocks (batch * H_kv * ceil(G * L / R), R as
 * for the balanced schedule) and piece states (num_splits * R * (head_dim
 * + 1) * 4 bytes, ~3.2 MB for 64 requests with H_q 32, H_kv 8, D 128) that
 * fit in the rest of the array; a call beyond them, or one whose plan is
 * the partition schedule (batch above 2048), returns PA_ERR_SCRATCH and
 * enqueues nothing.  All calls on one GPU share that GPU's array: calls
 * that overlap in time on one GPU (different streams without ordering, or
 * different host threads) race and give undefined results. */
pa_status pa_decode_noalloc(const pa_args *args, void *stream);

/* Static description of a status code (never NULL). */
const char *pa_status_string(int32_t status);

/* PA_ABI_VERSION of the built library. */
int32_t pa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
