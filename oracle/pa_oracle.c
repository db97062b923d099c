/*
 * CPU oracle for the paged-attention read path.  TEST INFRASTRUCTURE ONLY:
 * tests, the smoke check and the benchmark's CPU-baseline leg call it; the
 * product path never does.  It shares no code with the GPU library.
 *
 * What it computes is the plain definition.  Paging only changes where K/V
 * live, never what attention computes ("Reading vLLM's PagedAttention Kernel",
 * sections 2 and 4, and its pitfall list in section 6), so the oracle
 *   1. translates every logical key position j of request b through the block
 *      table: logical page j / page_size -> physical page block_table[b][j /
 *      page_size] -> slot j % page_size  (tiny-llm "Week 3 Day 4", sections
 *      "Why block_table Matters" and "How This Maps to tiny-llm");
 *   2. gathers the visible K/V rows of one (request, kv head) into a dense
 *      array, taking only the first context_lens[b] tokens (anllm "Tutorial
 *      13", section 5, gather_dense over valid page prefixes);
 *   3. runs ordinary two-pass softmax attention on the dense rows:
 *      s_j = scale * q . k_j, m = max s_j, w_j = exp(s_j - m),
 *      o = sum_j w_j v_j / sum_j w_j  (the dense_attention reference of
 *      "Reading vLLM's PagedAttention Kernel", section 4).
 * Precision: the arithmetic type `real` is float when the file is built
 * with -DOR_SINGLE (the plain fp32 two-pass reference: fp32 products, sums,
 * expf and logf) and double otherwise (the stricter check: the same steps
 * in fp64).  bf16 and fp32 inputs are widened exactly; results are handed
 * back as double arrays in both builds.
 *
 * Readings where the pages leave a step open:
 *   - query head h reads kv head h / (H_q / H_kv) (contiguous GQA groups);
 *   - causal rows are bottom-right aligned: row i of request b sits at
 *     position qpos = context_lens[b] - query_lens[b] + i and sees keys
 *     j <= qpos (K/V of the new rows are appended before attention, tiny-llm
 *     "Decode Metadata" / "Task 3");
 *   - rows i >= query_lens[b] and rows with no visible key produce zeros;
 *   - split partitions cover tokens [s*P, min((s+1)*P, ctx)); an empty one has
 *     o = 0 and lse = -inf; partitions merge by log-sum-exp weights
 *     ("Reading vLLM's PagedAttention Kernel", section 3.3, PARTITION_SIZE).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum {
  OR_OK = 0,
  OR_BAD_SHAPE = 1,   /* a size or a divisibility rule is violated */
  OR_BAD_PAGE = 2,    /* a block-table entry that must be read is out of range */
  OR_BAD_CTX = 3,     /* context_lens[b] < 0 or > max_pages * page_size */
  OR_BAD_QLEN = 4,    /* query_lens[b] < 0, > L, or (causal) > context_lens[b] */
  OR_NOMEM = 5
};
enum { OR_F32 = 0, OR_BF16 = 1, OR_FP8E4M3 = 2 };

#ifdef OR_SINGLE
typedef float real;
#define R_EXP expf
#define R_LOG logf
#define R_INF INFINITY
#else
typedef double real;
#define R_EXP exp
#define R_LOG log
#define R_INF INFINITY
#endif

typedef struct {
  const void *q, *kp, *vp;
  const int32_t *bt, *cl, *ql;
  int B, Hq, Hkv, L, D, num_pages, page_size, max_pages, dtype, causal;
  double scale;
  int kv_dtype;            /* element type of the pages: OR_F32, OR_BF16 or OR_FP8E4M3 */
  double k_scale, v_scale; /* fp8 pages: stored code times scale is the value */
} or_args;

static real widen(const void *base, size_t idx, int dtype) {
  if (dtype == OR_F32) return (real)((const float *)base)[idx];
  uint32_t bits = ((uint32_t)((const uint16_t *)base)[idx]) << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (real)f;
}

/* Value of an 8-bit float in the OCP E4M3 encoding ("Reading vLLM's
 * PagedAttention Kernel", section 3.2: the cache write takes a kv-cache dtype
 * and per-tensor k/v scales; the reading of the fp8 variant is the OCP
 * 8-bit format with 4 exponent and 3 mantissa bits): bit 7 sign, bits 6..3
 * exponent e with bias 7, bits 2..0 mantissa m.  e >= 1 is the normal value
 * (1 + m/8) 2^(e-7); e = 0 is the subnormal value (m/8) 2^-6; the pattern
 * with every exponent and mantissa bit set is NaN, and there is no
 * infinity. */
static real e4m3_value(uint8_t code) {
  const int sign = code >> 7, e = (code >> 3) & 15, m = code & 7;
  if (e == 15 && m == 7) return (real)NAN;
  const real mag = e == 0 ? (real)ldexp((double)m, -9) : (real)ldexp((double)(8 + m), e - 10);
  return sign ? -mag : mag;
}

/* Element idx of a page pool: its stored value, dequantised for fp8 pages
 * (code value times the pool's scale). */
static real page_value(const or_args *a, const void *pool, size_t idx, double kv_scale) {
  if (a->kv_dtype == OR_FP8E4M3)
    return e4m3_value(((const uint8_t *)pool)[idx]) * (real)kv_scale;
  return widen(pool, idx, a->kv_dtype);
}

static int qlen_of(const or_args *a, int b) { return a->ql ? a->ql[b] : a->L; }

/* Validate shapes and the caller's side of the contract (which the GPU path
 * takes on trust in release builds). */
static int check(const or_args *a) {
  if (a->B < 0 || a->Hq <= 0 || a->Hkv <= 0 || a->L <= 0 || a->D <= 0 ||
      a->page_size <= 0 || a->max_pages <= 0 || a->num_pages <= 0)
    return OR_BAD_SHAPE;
  if (a->Hq % a->Hkv != 0) return OR_BAD_SHAPE;
  if (!(a->scale > 0.0) || !isfinite(a->scale)) return OR_BAD_SHAPE;
  if (a->kv_dtype != OR_F32 && a->kv_dtype != OR_BF16 && a->kv_dtype != OR_FP8E4M3)
    return OR_BAD_SHAPE;
  if (a->kv_dtype == OR_FP8E4M3 && (!(a->k_scale > 0.0) || !isfinite(a->k_scale) ||
                                    !(a->v_scale > 0.0) || !isfinite(a->v_scale)))
    return OR_BAD_SHAPE;
  for (int b = 0; b < a->B; ++b) {
    int ctx = a->cl[b];
    if (ctx < 0 || (int64_t)ctx > (int64_t)a->max_pages * a->page_size) return OR_BAD_CTX;
    int n_pages = (ctx + a->page_size - 1) / a->page_size;
    for (int lp = 0; lp < n_pages; ++lp) {
      int p = a->bt[(size_t)b * a->max_pages + lp];
      if (p < 0 || p >= a->num_pages) return OR_BAD_PAGE;
    }
    int lq = qlen_of(a, b);
    if (lq < 0 || lq > a->L) return OR_BAD_QLEN;
    if (a->causal && lq > ctx) return OR_BAD_QLEN;
  }
  return OR_OK;
}

/* Step 1: logical key j of request b -> (physical page, slot). */
static void translate(const or_args *a, int b, int j, int *page, int *slot) {
  int lp = j / a->page_size;
  *slot = j - lp * a->page_size;
  *page = a->bt[(size_t)b * a->max_pages + lp];
}

/* Step 2: dense copies of the first ctx keys/values of (b, kv head g). */
static void gather_dense(const or_args *a, int b, int g, real *Kd, real *Vd) {
  const int ctx = a->cl[b], D = a->D;
  for (int j = 0; j < ctx; ++j) {
    int page, slot;
    translate(a, b, j, &page, &slot);
    size_t base = (((size_t)page * a->Hkv + g) * a->page_size + slot) * (size_t)D;
    for (int d = 0; d < D; ++d) {
      Kd[(size_t)j * D + d] = page_value(a, a->kp, base + d, a->k_scale);
      Vd[(size_t)j * D + d] = page_value(a, a->vp, base + d, a->v_scale);
    }
  }
}

/* Step 3: two-pass softmax attention of one query row over dense keys
 * [lo, hi).  Writes o[D]; returns the log-sum-exp of the scaled scores
 * (-inf when the span is empty, with o = 0). */
static real dense_attention(const or_args *a, const real *q, const real *Kd, const real *Vd,
                            int lo, int hi, real *s, real *o) {
  const int D = a->D;
  const real scale = (real)a->scale;
  for (int d = 0; d < D; ++d) o[d] = 0;
  if (hi <= lo) return -R_INF;
  real m = -R_INF;
  for (int j = lo; j < hi; ++j) {
    real acc = 0;
    for (int d = 0; d < D; ++d) acc += q[d] * Kd[(size_t)j * D + d];
    s[j] = scale * acc;
    if (s[j] > m) m = s[j];
  }
  real Z = 0;
  for (int j = lo; j < hi; ++j) {
    real w = R_EXP(s[j] - m);
    Z += w;
    for (int d = 0; d < D; ++d) o[d] += w * Vd[(size_t)j * D + d];
  }
  for (int d = 0; d < D; ++d) o[d] /= Z;
  return m + R_LOG(Z);
}

/* Visible key limit of row i of request b. */
static int row_limit(const or_args *a, int b, int i) {
  int ctx = a->cl[b];
  if (!a->causal) return ctx;
  return ctx - qlen_of(a, b) + i + 1;
}

/* Shared loop: for every (b, g) gather densely, then for every query row of
 * the group compute either the full result (P <= 0) or S partition states. */
static int run(const or_args *a, int P, int S, double *out, double *part_o,
               double *part_lse, int nthreads, int *threads_used) {
  int rc = check(a);
  if (rc) return rc;
  const int G = a->Hq / a->Hkv, D = a->D, L = a->L;
  int max_ctx = 0;
  for (int b = 0; b < a->B; ++b)
    if (a->cl[b] > max_ctx) max_ctx = a->cl[b];
  const size_t rows = (size_t)a->B * a->Hq * L;
  if (out) memset(out, 0, rows * D * sizeof(double));
  if (part_o) memset(part_o, 0, rows * (size_t)S * D * sizeof(double));
  if (part_lse)
    for (size_t r = 0; r < rows * (size_t)S; ++r) part_lse[r] = -INFINITY;
  int failed = 0, used = 1;
  const int units = a->B * a->Hkv;
#pragma omp parallel num_threads(nthreads > 0 ? nthreads : 1) reduction(| : failed)
  {
#ifdef _OPENMP
#pragma omp single
    used = omp_get_num_threads();
#endif
    size_t n = (size_t)(max_ctx > 0 ? max_ctx : 1);
    real *Kd = malloc(n * D * sizeof(real));
    real *Vd = malloc(n * D * sizeof(real));
    real *s = malloc(n * sizeof(real));
    real *q = malloc((size_t)D * sizeof(real));
    real *o = malloc((size_t)D * sizeof(real));
    if (!Kd || !Vd || !s || !q || !o) failed = 1;
#pragma omp for schedule(dynamic, 1)
    for (int u = 0; u < units; ++u) {
      if (failed) continue;
      const int b = u / a->Hkv, g = u % a->Hkv;
      gather_dense(a, b, g, Kd, Vd);
      const int lq = qlen_of(a, b);
      for (int hh = 0; hh < G; ++hh) {
        const int h = g * G + hh;
        for (int i = 0; i < lq; ++i) {
          const size_t row = ((size_t)b * a->Hq + h) * L + i;
          for (int d = 0; d < D; ++d) q[d] = widen(a->q, row * D + d, a->dtype);
          const int hi = row_limit(a, b, i);
          if (P <= 0) {
            dense_attention(a, q, Kd, Vd, 0, hi, s, o);
            for (int d = 0; d < D; ++d) out[row * D + d] = (double)o[d];
          } else {
            for (int sp = 0; sp < S; ++sp) {
              int lo = sp * P, e = lo + P;
              if (e > hi) e = hi;
              real lse = dense_attention(a, q, Kd, Vd, lo, e, s, o);
              part_lse[row * S + sp] = (double)lse;
              for (int d = 0; d < D; ++d) part_o[(row * S + sp) * D + d] = (double)o[d];
            }
          }
        }
      }
    }
    free(Kd); free(Vd); free(s); free(q); free(o);
  }
  if (threads_used) *threads_used = used;
  return failed ? OR_NOMEM : OR_OK;
}

#define ARGS_DECL                                                                      \
  const void *q, const void *kp, const void *vp, const int32_t *bt, const int32_t *cl, \
      const int32_t *ql, int B, int Hq, int Hkv, int L, int D, int num_pages,          \
      int page_size, int max_pages, int dtype, int causal, double scale, int kv_dtype,   \
      double k_scale, double v_scale
#define ARGS_INIT                                                                     \
  or_args a = {q, kp, vp, bt, cl, ql, B, Hq, Hkv, L, D, num_pages, page_size, max_pages, \
               dtype, causal, scale, kv_dtype, k_scale, v_scale}

/* Full attention: out[B][Hq][L][D] (double). */
int or_attention(ARGS_DECL, int nthreads, int *threads_used, double *out) {
  ARGS_INIT;
  return run(&a, 0, 0, out, NULL, NULL, nthreads, threads_used);
}

/* Per-partition states: part_o[B][Hq][L][S][D], part_lse[B][Hq][L][S]. */
int or_partials(ARGS_DECL, int partition_tokens, int num_splits, int nthreads,
                double *part_o, double *part_lse) {
  ARGS_INIT;
  if (partition_tokens <= 0 || num_splits <= 0) return OR_BAD_SHAPE;
  return run(&a, partition_tokens, num_splits, NULL, part_o, part_lse, nthreads, NULL);
}

/* Log-sum-exp merge of S partition states per row:
 *   M = max_s lse_s, w_s = exp(lse_s - M) / sum_t exp(lse_t - M),
 *   out = sum_s w_s o_s; a row whose partitions are all empty gets 0. */
int or_merge(const double *part_o, const double *part_lse, long rows, int S, int D,
             double *out) {
  real *o = malloc((size_t)(D > 0 ? D : 1) * sizeof(real));
  if (!o) return OR_NOMEM;
  for (long r = 0; r < rows; ++r) {
    real M = -R_INF;
    for (int s = 0; s < S; ++s)
      if ((real)part_lse[r * S + s] > M) M = (real)part_lse[r * S + s];
    for (int d = 0; d < D; ++d) o[d] = 0;
    if (M != -R_INF) {
      real Z = 0;
      for (int s = 0; s < S; ++s) Z += R_EXP((real)part_lse[r * S + s] - M);
      for (int s = 0; s < S; ++s) {
        real w = R_EXP((real)part_lse[r * S + s] - M) / Z;
        if (w == 0) continue;
        const double *os = part_o + ((size_t)r * S + s) * D;
        for (int d = 0; d < D; ++d) o[d] += w * (real)os[d];
      }
    }
    for (int d = 0; d < D; ++d) out[(size_t)r * D + d] = (double)o[d];
  }
  free(o);
  return OR_OK;
}

/* Address trace: trace[b][j] = (physical page, slot) for j < context_lens[b],
 * (-1, -1) beyond; trace has B * max_pages * page_size * 2 int32. */
int or_translate(const int32_t *bt, const int32_t *cl, int B, int max_pages, int page_size,
                 int num_pages, int32_t *trace) {
  or_args a;
  memset(&a, 0, sizeof a);
  a.bt = bt; a.cl = cl; a.B = B; a.max_pages = max_pages; a.page_size = page_size;
  a.num_pages = num_pages; a.Hq = a.Hkv = a.L = a.D = 1; a.scale = 1.0;
  a.kv_dtype = OR_F32;
  int rc = check(&a);
  if (rc) return rc;
  const size_t cap = (size_t)max_pages * page_size;
  for (int b = 0; b < B; ++b)
    for (size_t j = 0; j < cap; ++j) {
      int32_t *t = trace + ((size_t)b * cap + j) * 2;
      if ((int)j < cl[b]) {
        int page, slot;
        translate(&a, b, (int)j, &page, &slot);
        t[0] = page; t[1] = slot;
      } else {
        t[0] = -1; t[1] = -1;
      }
    }
  return OR_OK;
}

/* The value of each of n fp8 E4M3 codes (for pins of the decoder). */
int or_e4m3_values(const uint8_t *codes, long n, double *out) {
  for (long i = 0; i < n; ++i) out[i] = (double)e4m3_value(codes[i]);
  return OR_OK;
}
