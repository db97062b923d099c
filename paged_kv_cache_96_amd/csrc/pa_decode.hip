// Paged decode kernel (vector ALU) for gfx950, with split-KV partitions.
//
// Schedule (tiny-llm "Week 3 Day 4", "Choose a Schedule for Each Query Shape"
// and "Checkpoint 2": parallelise short queries across the cached context,
// coalesce lanes over head elements, resolve a page id once per page, keep
// the query and the softmax state in registers, reduce with cross-lane
// operations; "Reading vLLM's PagedAttention Kernel" section 3.3: split long
// contexts into partitions that are merged afterwards):
//
//   Work item = partition s of the ROWS packed query rows (row rho ->
//   position rho / G, head g*G + rho % G) of kv head g of request b; one
//   wave owns an item, so each K/V byte of the partition is read once for
//   all of those rows, and the waves of a workgroup run independently (no
//   barrier or LDS merge per item).  The wave walks the partition in steps
//   of STEP keys.  In a step every lane issues 16-byte loads: LPT
//   lanes cover one key's D elements and a wave load covers TPL keys, so the
//   loads of a page are fully coalesced.  K/V are read exactly once, with
//   non-temporal loads.
//
//   Page resolution: when steps never straddle a page (page_size a multiple
//   of STEP) each wave computes the 64-bit element offset of the page/slot of
//   each of its steps once, up front, one step per lane; the walk then takes
//   the offset of step k with a readlane, so the loop issues no memory
//   operation besides the K/V loads and addresses are formed in scalar
//   registers.  Other page sizes resolve the page per lane.
//
//   Softmax state: every group of LPT lanes (one key of each load) keeps its
//   own running max / sum / output for every row, so the walk needs no
//   cross-group exchange.  The max is refreshed lazily: only when a new score
//   exceeds the reference max by more than 2^8 (the weights then stay below
//   256 and fp32 sums stay exact to rounding).  Dot products are summed over
//   the LPT lanes with DPP; scores are kept in base-2 units.  For bf16 the
//   PV product runs on bf16 dot2 instructions with the weights rounded to
//   bf16 (two keys per instruction), and the row sums add those same rounded
//   weights.  At the end the lane groups are merged in registers and the
//   partition state is written (normalised output plus log-sum-exp), or the
//   final output when there is one partition.
//
//   fp8 pages (E4M3 codes with per-tensor k/v scales, bf16 query and output):
//   a lane's 16-byte load holds 16 elements of one key, so a wave load covers
//   8 keys (D = 128) and a step 32; every pair of codes is widened exactly
//   to a bf16 pair (v_cvt_scalef32_pk_bf16_fp8 with scale 1) and the
//   arithmetic is that of bf16 pages.  k_scale folds into the score multiplier, v_scale into the
//   final division.  A step spans two 16-key halves, each resolved to its
//   own page, so 16-key pages keep the page-uniform walk.
#include <type_traits>

#include "pa_common.hpp"
#include "pa_internal.h"
#include "pa_merge.hpp"

namespace pa {
namespace {

using Vec = u32x4_t;  // one 16-byte lane load (the type buffer loads return)


constexpr float kMinM = -1.0e30f;  // running-max sentinel: exp2(x - kMinM) never overflows
// Register buffers of the page-uniform walk (kDecodeBuffers - 1 steps in
// flight while one is folded).
constexpr int kDecodeBuffers = 3;


constexpr float kLazy = 8.0f;      // refresh the max only when it grows by more than this (log2)

template <typename T>
struct Elem;
template <>
struct Elem<float> {
  static constexpr int kPerVec = 4;
};
template <>
struct Elem<uint16_t> {
  static constexpr int kPerVec = 8;
};
template <>
struct Elem<uint8_t> {
  static constexpr int kPerVec = 16;
};

template <typename T>
__device__ __forceinline__ void widen(const Vec &v, float (&f)[Elem<T>::kPerVec]) {
  if constexpr (sizeof(T) == 4) {
    f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
  } else {
    f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x); f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
    f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z); f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
  }
}

// Partial q.k over this lane's elements.
template <typename T>
__device__ __forceinline__ float lane_dot(const Vec &q, const Vec &k) {
  if constexpr (sizeof(T) == 4) {
    float a = __uint_as_float(q.x) * __uint_as_float(k.x);
    a = fmaf(__uint_as_float(q.y), __uint_as_float(k.y), a);
    a = fmaf(__uint_as_float(q.z), __uint_as_float(k.z), a);
    return fmaf(__uint_as_float(q.w), __uint_as_float(k.w), a);
  } else {
    float a = dot2_bf16(q.x, k.x, 0.f);
    a = dot2_bf16(q.y, k.y, a);
    a = dot2_bf16(q.z, k.z, a);
    return dot2_bf16(q.w, k.w, a);
  }
}

__device__ __forceinline__ uint32_t word(const Vec &v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// The elements of a lane's page load as bf16 pairs: pair j holds elements
// 2j and 2j + 1.  bf16 pages: the loaded words.  fp8 pages: every code
// widened exactly (an E4M3 value is a bf16 value) by the hardware converter
// of two codes to a bf16 pair, with scale 1 (its results match the
// format's definition for all 256 codes, checked on the device).
template <typename KV>
__device__ __forceinline__ void to_pairs(const Vec &v, uint32_t (&pr)[Elem<KV>::kPerVec / 2]) {
  if constexpr (sizeof(KV) == 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t w = word(v, i);
      pr[2 * i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(
                                                   w, 1.0f, false));  // bytes 0, 1
      pr[2 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(
                                                       w, 1.0f, true));  // bytes 2, 3
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) pr[i] = word(v, i);
  }
}

// Scan of v over the 256 threads of a workgroup in thread order with the
// associative `op` (identity `id`): lane shifts within each wave, then the
// four wave totals through s_w (one barrier).  Returns the inclusive value
// and sets *excl to the exclusive one.  s_w may be reused once every thread
// has passed a later barrier.
template <typename Op>
__device__ __forceinline__ long long block_scan(long long v, long long id, Op op, long long *s_w,
                                                long long *excl) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const long long n = __shfl_up(v, off, 64);
    if (lane >= off) v = op(v, n);
  }
  if (lane == 63) s_w[wv] = v;
  __syncthreads();
  long long pre = id;
  for (int k = 0; k < wv; ++k) pre = op(pre, s_w[k]);
  const long long up = __shfl_up(v, 1, 64);
  *excl = op(pre, lane > 0 ? up : id);
  return op(pre, v);
}

// Where a work item's state goes.  Partition schedule: slot `slot` of each
// row.  Balanced schedule: piece slot `piece` of the row block, whose
// `pieces` pieces occupy slots first, first + 1, ...; with arrival counters
// the last piece to finish merges them (counter `unit`).
struct ItemOut {
  int slot;
  long long piece;  // < 0: partition schedule
  long long first;
  int pieces;
  long long unit;
};

// One work item, walked by the calling wave alone: keys [t0, tend) of the
// ROWS-row block rb of kv head g of request b (t0 a multiple of STEP).
// With `split` it writes the state of that piece to the workspace (see
// ItemOut), otherwise the piece is the whole row range and it writes the
// output.
// With `pre` (a request of a shared-prefix group; split then holds) the
// fused merge starts every row from the row's prefix state.
template <typename T, typename KV, int D, int ROWS, bool DEBUG, bool UNIFORM>
__device__ __forceinline__ void decode_item(const LaunchParams &p, int b, int g, int rb, int t0,
                                            int tend, const ItemOut &io, bool split, int ctx,
                                            int Lb, int q0, bool pre = false) {
  constexpr bool kFp8 = sizeof(KV) == 1;  // fp8 E4M3 pages (T: bf16)
  constexpr int kElems = Elem<KV>::kPerVec;  // page elements per 16-byte lane load
  constexpr int kLpt = D / kElems;      // lanes per key
  constexpr int kTpl = 64 / kLpt;       // keys per wave load
  constexpr int kLoads = 4;             // loads in flight per step (each of K and V)
  constexpr int kStep = kTpl * kLoads;  // keys per wave step
  constexpr int kResKeys = kFp8 ? 16 : kStep;  // keys resolved to one page at a time
  constexpr int kRes = kStep / kResKeys;       // page resolutions per step
  constexpr int kLoadsPerRes = kLoads / kRes;
  constexpr int kPairs = kElems / 2;    // bf16 pairs per lane load (dot2 paths)
  constexpr int kQVecs = kElems * (int)sizeof(T) / 16;  // 16-byte query pieces per lane
  constexpr int kBuf = kDecodeBuffers;  // rotating register buffers of the walk
  constexpr bool kBf16 = sizeof(T) == 2;  // bf16 query: dot2 arithmetic
  static_assert(kLpt * kElems == D && kTpl * kLpt == 64, "layout");
  static_assert(kRes * kResKeys == kStep && kLoadsPerRes * kRes == kLoads, "resolutions");
  static_assert(!kFp8 || kBf16, "fp8 pages take a bf16 query");
  const int lane = threadIdx.x & 63;
  const int c = lane % kLpt;            // element chunk of this lane
  const int kl = lane / kLpt;           // key of this lane within a load

  const int G = p.Hq / p.Hkv;
  const int ps = p.ps;
  const int32_t *bt = p.bt + (size_t)b * p.max_pages;

  // ---- rows of this workgroup
  int hi[ROWS];
  bool valid[ROWS];
  size_t qrow[ROWS];
  int kmax = 0, kmin = 0x7fffffff;
#pragma unroll
  for (int r = 0; r < ROWS; ++r) {
    const int rho = rb * ROWS + r;
    const int i = rho / G;
    const int h = g * G + (rho - i * G);
    valid[r] = rho < G * p.L && i < Lb;
    hi[r] = valid[r] ? (p.causal ? ctx - Lb + i + 1 : ctx) : 0;
    // packed rows: q0 is the request's first row (query_start_loc[b])
    qrow[r] = p.qsl ? (size_t)(q0 + i) * p.Hq + h : query_row(p, b, h, i);
    kmax = max(kmax, hi[r]);
    if (valid[r]) kmin = min(kmin, hi[r]);
  }
  const int t1 = min(tend, kmax);
  // the row block holding the last packed row of the request counts visits
  const bool counts = DEBUG && Lb > 0 && ((Lb * G - 1) / ROWS == rb);

  Vec qv[ROWS][kQVecs];
  const T *qbase = reinterpret_cast<const T *>(p.q);
#pragma unroll
  for (int r = 0; r < ROWS; ++r) {
    // padded rows past query_lens are in bounds (i < L): load unconditionally,
    // then drop; packed rows past the request's own do not exist
    const bool exists = p.qsl ? valid[r] : rb * ROWS + r < G * p.L;
#pragma unroll
    for (int v = 0; v < kQVecs; ++v) {
      const Vec x = exists ? *reinterpret_cast<const Vec *>(qbase + qrow[r] * D + c * kElems +
                                                            v * (16 / (int)sizeof(T)))
                           : Vec{0u, 0u, 0u, 0u};
      qv[r][v] = valid[r] ? x : Vec{0u, 0u, 0u, 0u};
    }
  }
  // query word j of row r (bf16 pair of elements 2j, 2j + 1 of the lane)
  auto qword = [&](int r, int j) { return word(qv[r][j / 4], j % 4); };

  float m[ROWS], l[ROWS], acc[ROWS][kElems];
#pragma unroll
  for (int r = 0; r < ROWS; ++r) {
    m[r] = kMinM;
    l[r] = 0.f;
#pragma unroll
    for (int e = 0; e < kElems; ++e) acc[r][e] = 0.f;
  }

  const KV *kp = reinterpret_cast<const KV *>(p.kp);
  const KV *vp = reinterpret_cast<const KV *>(p.vp);
  const int nsteps = t1 > t0 ? (t1 - t0 + kStep - 1) / kStep : 0;
  const int nw = nsteps;  // steps of this wave
  const int tmin = min(t1, kmin);  // keys below this are visible to every valid row
  // leading steps that lie wholly below tmin (no key of them is masked)
  const int nfull = tmin > t0 ? min(nw, (tmin - t0) / kStep) : 0;
  const size_t head_stride = (size_t)ps * D;
  const uint32_t lane_off = (uint32_t)(kl * D + c * kElems);

  // Offsets of the page/slot of this wave's steps k0 .. k0+63 (one step per
  // lane; kRes resolutions of kResKeys keys each per step).  Only keys below
  // t1 are resolved: block-table entries past the context are never read.
  uint32_t off_lo[kRes], off_hi[kRes];
#pragma unroll
  for (int rr = 0; rr < kRes; ++rr) off_lo[rr] = off_hi[rr] = 0u;
  auto resolve = [&](int k0) {
    const int k = k0 + lane;
#pragma unroll
    for (int rr = 0; rr < kRes; ++rr) {
      const int base = t0 + k * kStep + rr * kResKeys;
      if (k < nw && base < t1) {
        const int lp = base / ps;
        const int page = bt[lp];
        const size_t off =
            ((size_t)page * p.Hkv + g) * head_stride + (size_t)(base - lp * ps) * D;
        off_lo[rr] = (uint32_t)off;
        off_hi[rr] = (uint32_t)(off >> 32);
      }
    }
  };

  // Debug record of logical key j, decoded from the element offset `eoff`
  // that this lane's load of the key actually uses (its first 16-byte chunk:
  // c == 0): physical page, slot and kv head follow from the pool layout
  // [num_pages, H_kv, page_size, D] alone, so the trace observes the address
  // arithmetic of the walk rather than restating it.  The visit is counted
  // under the kv head the offset points at.
  auto record = [&](int j, size_t eoff) {
    if constexpr (DEBUG) {
      if (counts && c == 0 && j < t1) {
        const size_t row = eoff / D;            // (page * H_kv + head) * ps + slot
        const size_t ph = row / (size_t)ps;     // page * H_kv + head
        const int slot = (int)(row - ph * ps);
        const int page = (int)(ph / p.Hkv);
        const int head = (int)(ph - (size_t)page * p.Hkv);
        const size_t cap = (size_t)p.max_pages * ps;
        if (g == 0) {
          p.dbg_trace[((size_t)b * cap + j) * 2 + 0] = page;
          p.dbg_trace[((size_t)b * cap + j) * 2 + 1] = slot;
        }
        atomicAdd(&p.dbg_visits[((size_t)b * p.Hkv + head) * cap + j], 1);
      }
    }
  };

  // Element offset of key n*TPL + kl of step k, resolved per lane (page
  // sizes that are not a multiple of the step).
  auto key_offset = [&](int k, int n) -> size_t {
    int j = t0 + k * kStep + n * kTpl + kl;
    j = min(j, t1 - 1);  // keys past the end reuse a valid address; masked below
    const int lp = j / ps;
    const int page = bt[lp];
    const int slot = j - lp * ps;
    return ((size_t)page * p.Hkv + g) * head_stride + (size_t)slot * D + c * kElems;
  };

  auto load_step = [&](int k, Vec (&kv)[kLoads], Vec (&vv)[kLoads]) {
#pragma unroll
    for (int n = 0; n < kLoads; ++n) {
      const size_t off = key_offset(k, n);
      kv[n] = load_stream(kp + off);
      vv[n] = load_stream(vp + off);
      record(t0 + k * kStep + n * kTpl + kl, off);
    }
  };

  // Steps of a uniform walk are fetched through buffer resources whose base
  // is the step's page/slot: a step past the end gets num_records = 0, so its
  // loads return zeros without touching memory.  Every fetch is then issued
  // unconditionally, and the compiler's wait counts see a straight-line
  // stream of loads (with conditional fetches it must assume the later loads
  // may be missing and waits for them too, which serialises the pipeline).
  auto fetch_uniform = [&](auto refresh, int k, Vec (&kv)[kLoads], Vec (&vv)[kLoads]) {
    const bool ok = k < nw;
    if constexpr (decltype(refresh)::value) {
      if (k > 0 && (k & 63) == 0 && ok) resolve(k);
    }
#pragma unroll
    for (int rr = 0; rr < kRes; ++rr) {
      const uint32_t lo = __builtin_amdgcn_readlane(off_lo[rr], k & 63);
      const uint32_t hi2 = __builtin_amdgcn_readlane(off_hi[rr], k & 63);
      const size_t base = ((size_t)hi2 << 32) | lo;
      const bool live = ok && t0 + k * kStep + rr * kResKeys < t1;  // wave-uniform
      const int nrec = live ? kResKeys * D * (int)sizeof(KV) : 0;
      const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<KV *>(kp + base), (short)0, nrec, kBufferRsrcWord3);
      const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<KV *>(vp + base), (short)0, nrec, kBufferRsrcWord3);
#pragma unroll
      for (int nn = 0; nn < kLoadsPerRes; ++nn) {
        const int n = rr * kLoadsPerRes + nn;
        const int boff = (int)((lane_off + nn * kTpl * D) * sizeof(KV));
        kv[n] = load_stream_buf(rk, boff);
        vv[n] = load_stream_buf(rv, boff);
        // the resource base plus the lane's byte offset, in elements
        if (live) record(t0 + k * kStep + n * kTpl + kl, base + (size_t)boff / sizeof(KV));
      }
    }
  };

  // score multiplier in base-2 units (fp8 pages: times k_scale)
  const float cs = kFp8 ? p.scale_log2 * p.k_scale : p.scale_log2;
  // `maybe_tail`: the step may hold keys at or past some row's limit (masked
  // scores, stale slots); false for the steps below tmin, whose fold then
  // carries no masking code at all.
  auto fold_step = [&](auto maybe_tail, int k, const Vec (&kv)[kLoads], const Vec (&vv)[kLoads]) {
    const int base = t0 + k * kStep;
    const bool tail = decltype(maybe_tail)::value && base + kStep > tmin;
    float sc[kLoads][ROWS];
#pragma unroll
    for (int n = 0; n < kLoads; ++n) {
      if constexpr (kBf16) {
        uint32_t kpr[kPairs];
        to_pairs<KV>(kv[n], kpr);
#pragma unroll
        for (int r = 0; r < ROWS; ++r) {
          float a = 0.f;
#pragma unroll
          for (int j = 0; j < kPairs; ++j) a = dot2_bf16(qword(r, j), kpr[j], a);
          sc[n][r] = group_sum<kLpt>(a);
        }
      } else {
#pragma unroll
        for (int r = 0; r < ROWS; ++r) sc[n][r] = group_sum<kLpt>(lane_dot<T>(qv[r][0], kv[n]));
      }
    }
    if (tail) {
#pragma unroll
      for (int n = 0; n < kLoads; ++n) {
        const int j = base + n * kTpl + kl;
#pragma unroll
        for (int r = 0; r < ROWS; ++r)
          if (j >= min(hi[r], t1)) sc[n][r] = kNegInf;
      }
    }
    // lazy refresh of the per-group reference max
    float mx[ROWS];
    bool need = false;
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
      float v = sc[0][r];
#pragma unroll
      for (int n = 1; n < kLoads; ++n) v = fmaxf(v, sc[n][r]);
      mx[r] = v * cs;
      need |= mx[r] > m[r] + kLazy;
    }
    if (__builtin_amdgcn_ballot_w64(need) != 0) {
#pragma unroll
      for (int r = 0; r < ROWS; ++r) {
        const float mn = fmaxf(m[r], mx[r]);
        const float alpha = fast_exp2(m[r] - mn);
        m[r] = mn;
        l[r] *= alpha;
#pragma unroll
        for (int e = 0; e < kElems; ++e) acc[r][e] *= alpha;
      }
    }
#pragma unroll
    for (int n = 0; n < kLoads; ++n)
#pragma unroll
      for (int r = 0; r < ROWS; ++r) {
        const float pr = fast_exp2(fmaf(sc[n][r], cs, -m[r]));
        sc[n][r] = pr;
        if constexpr (!kBf16) l[r] += pr;
      }
    // stale slots past the context may hold anything, NaN included
    bool dead[kLoads];
#pragma unroll
    for (int n = 0; n < kLoads; ++n) dead[n] = tail && (base + n * kTpl + kl >= t1);
    if constexpr (kBf16) {
#pragma unroll
      for (int n = 0; n < kLoads; n += 2) {
        uint32_t pk[ROWS];
#pragma unroll
        for (int r = 0; r < ROWS; ++r) {
          pk[r] = cvt_pk_bf16(sc[n][r], sc[n + 1][r]);
          l[r] = dot2_bf16(pk[r], 0x3f803f80u, l[r]);  // + both rounded weights (bf16 1.0 pair)
        }
        uint32_t va[kPairs], vb[kPairs];
        to_pairs<KV>(vv[n], va);
        to_pairs<KV>(vv[n + 1], vb);
#pragma unroll
        for (int w = 0; w < kPairs; ++w) {
          const uint32_t a = dead[n] ? 0u : va[w];
          const uint32_t bb = dead[n + 1] ? 0u : vb[w];
          const uint32_t lo = __builtin_amdgcn_perm(bb, a, 0x05040100u);  // dim 2w of keys n, n+1
          const uint32_t hi2 = __builtin_amdgcn_perm(bb, a, 0x07060302u); // dim 2w+1
#pragma unroll
          for (int r = 0; r < ROWS; ++r) {
            acc[r][2 * w] = dot2_bf16(pk[r], lo, acc[r][2 * w]);
            acc[r][2 * w + 1] = dot2_bf16(pk[r], hi2, acc[r][2 * w + 1]);
          }
        }
      }
    } else {
#pragma unroll
      for (int n = 0; n < kLoads; ++n) {
        float vf[kElems];
        widen<T>(vv[n], vf);
#pragma unroll
        for (int e = 0; e < kElems; ++e) vf[e] = dead[n] ? 0.f : vf[e];
#pragma unroll
        for (int r = 0; r < ROWS; ++r)
#pragma unroll
          for (int e = 0; e < kElems; ++e) acc[r][e] = fmaf(sc[n][r], vf[e], acc[r][e]);
      }
    }
  };

  // ---- main walk over the partition's steps; kBuf register buffers
  // rotate so that the loads of the next kBuf - 1 steps are in flight while
  // a step is folded (the loop body is unrolled kBuf times for the rotation).
  Vec kbuf[kBuf][kLoads], vbuf[kBuf][kLoads];
  if constexpr (UNIFORM) {
    // A walk of at most 64 steps has every page offset resolved up
    // front; longer walks (a single partition over a long context) refresh
    // them every 64 steps.  The two loops are separate so that the refresh,
    // a vector load that must complete at once, never sits on a path of the
    // short loop (it would make the compiler wait for the prefetched loads).
    resolve(0);
    auto walk = [&](auto refresh) {
#pragma unroll
      for (int i = 0; i < kBuf - 1; ++i) fetch_uniform(refresh, i, kbuf[i], vbuf[i]);
      int k = 0;
      // straight-line bodies of kBuf whole steps: for fp8 pages first the
      // steps below tmin with no masking code (their fold is bound by its
      // vector work: 3% on C2-sized calls; bf16 pages measured no gain),
      // then the rest
      for (; kFp8 && k + kBuf <= nfull; k += kBuf) {
#pragma unroll
        for (int i = 0; i < kBuf; ++i) {
          fetch_uniform(refresh, k + i + kBuf - 1, kbuf[(i + kBuf - 1) % kBuf],
                        vbuf[(i + kBuf - 1) % kBuf]);
          fold_step(std::false_type(), k + i, kbuf[i], vbuf[i]);
        }
      }
      for (; k + kBuf <= nw; k += kBuf) {
#pragma unroll
        for (int i = 0; i < kBuf; ++i) {
          fetch_uniform(refresh, k + i + kBuf - 1, kbuf[(i + kBuf - 1) % kBuf],
                        vbuf[(i + kBuf - 1) % kBuf]);
          fold_step(std::true_type(), k + i, kbuf[i], vbuf[i]);
        }
      }
#pragma unroll
      for (int i = 0; i < kBuf - 1; ++i)  // the last (at most kBuf - 1) steps
        if (k + i < nw) fold_step(std::true_type(), k + i, kbuf[i], vbuf[i]);
    };
    if (nw <= 64) {
      walk(std::integral_constant<bool, false>());
    } else {
      walk(std::integral_constant<bool, true>());
    }
  } else if (nw > 0) {
    auto fetch = [&](int k, Vec (&kv)[kLoads], Vec (&vv)[kLoads]) {
      if (k < nw) load_step(k, kv, vv);
    };
    Vec (&ka)[kLoads] = kbuf[0], (&va)[kLoads] = vbuf[0];
    Vec (&kb)[kLoads] = kbuf[1], (&vb)[kLoads] = vbuf[1];
    Vec (&kc)[kLoads] = kbuf[2], (&vc)[kLoads] = vbuf[2];
    fetch(0, ka, va);
    fetch(1, kb, vb);
    for (int k = 0; k < nw; k += 3) {
      fetch(k + 2, kc, vc);
      fold_step(std::true_type(), k, ka, va);
      fetch(k + 3, ka, va);
      if (k + 1 < nw) fold_step(std::true_type(), k + 1, kb, vb);
      fetch(k + 4, kb, vb);
      if (k + 2 < nw) fold_step(std::true_type(), k + 2, kc, vc);
    }
  }

  // ---- merge the lane groups in registers, then write this partition
  T *out = reinterpret_cast<T *>(p.out);
  // rows written: padded rows up to G * L (past query_lens as zeros); packed
  // rows of the request only
  const int rows_out = p.qsl ? G * Lb : G * p.L;
#pragma unroll
  for (int r = 0; r < ROWS; ++r) {
    const float M = stride_max<kLpt>(m[r]);
    const float f = fast_exp2(m[r] - M);
    const float lt = stride_sum<kLpt>(l[r] * f);
#pragma unroll
    for (int e = 0; e < kElems; ++e) acc[r][e] = stride_sum<kLpt>(acc[r][e] * f);
    const int rho = rb * ROWS + r;
    if (rho >= rows_out) continue;  // a row that does not exist (or is not written)
    const bool has = valid[r] && lt > 0.f;
    // fp8 pages: the values carry v_scale, applied once here
    const float inv = has ? (kFp8 ? p.v_scale / lt : 1.f / lt) : 0.f;
    if (split) {
      if (!valid[r]) continue;  // the merge writes padding rows itself
      const size_t wi = io.piece >= 0 ? (size_t)io.piece * ROWS + r
                                      : qrow[r] * p.num_splits + io.slot;
      // written through to memory: a merging wave on another XCD reads them
      const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
          p.ws_o + wi * D, (short)0, D * 4, kBufferRsrcWord3);
      if (lane < kLpt) {
#pragma unroll
        for (int e = 0; e < kElems; e += 4) {
          const u32x4_t v = {__float_as_uint(acc[r][e] * inv), __float_as_uint(acc[r][e + 1] * inv),
                             __float_as_uint(acc[r][e + 2] * inv),
                             __float_as_uint(acc[r][e + 3] * inv)};
          __builtin_amdgcn_raw_buffer_store_b128(v, ro, (c * kElems + e) * 4, 0, kSysScope);
        }
      }
      if (lane == 0) {
        const __amdgpu_buffer_rsrc_t rl = __builtin_amdgcn_make_buffer_rsrc(
            p.ws_lse + wi, (short)0, 4, kBufferRsrcWord3);
        __builtin_amdgcn_raw_buffer_store_b32(
            __float_as_uint(has ? (M + __log2f(lt)) * kLn2 : kNegInf), rl, 0, 0, kSysScope);
      }
    } else if (lane < kLpt) {
      T *dst = out + qrow[r] * D + c * kElems;
      if constexpr (sizeof(T) == 4) {
        *reinterpret_cast<float4 *>(dst) =
            make_float4(acc[r][0] * inv, acc[r][1] * inv, acc[r][2] * inv, acc[r][3] * inv);
      } else {
#pragma unroll
        for (int e = 0; e < kElems; e += 8)
          *reinterpret_cast<uint4 *>(dst + e) =
              make_uint4(cvt_pk_bf16(acc[r][e] * inv, acc[r][e + 1] * inv),
                         cvt_pk_bf16(acc[r][e + 2] * inv, acc[r][e + 3] * inv),
                         cvt_pk_bf16(acc[r][e + 4] * inv, acc[r][e + 5] * inv),
                         cvt_pk_bf16(acc[r][e + 6] * inv, acc[r][e + 7] * inv));
      }
    }
  }

  // ---- fused merge (balanced schedule with arrival counters): the last
  // piece of the row block to arrive merges all of them into the output.
  // No wave waits for another: the arrival count decides who merges.
  if (split && io.piece >= 0 && p.counters != nullptr) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the states are in memory
    uint32_t *cnt = p.counters + io.unit;
    uint32_t old = 0;
    if (lane == 0) old = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    old = __builtin_amdgcn_readfirstlane(old);
    if (old == (uint32_t)(io.pieces - 1)) {
      asm volatile("" ::: "memory");
      const size_t wi = (size_t)io.first * ROWS;
      merge_block<T, D, ROWS>(p.ws_lse + wi, p.ws_o + wi * D, io.pieces, valid, qrow,
                              min(ROWS, rows_out - rb * ROWS), out, pre ? p.pre_lse : nullptr,
                              p.pre_o, p.pre_n);
      if (lane == 0) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// Decode kernel: four independent waves per workgroup, each walking its own
// work items.
//
// Partition schedule (p.balanced == 0): the grid names the items (x: wave
// index over partitions x (kv head x row block), the latter fastest; y:
// request); a wave owns partition s of one row block and exits at once when
// the partition is empty.
//
// Balanced schedule: the steps of every row block of every request are laid
// out request-major (request b, then unit u = kv head x row block, then the
// row block's ceil(context_len / STEP) steps) and the W active waves take
// equal contiguous runs of them: wave w owns [floor(w T / W), floor((w+1) T
// / W)).  A run crosses row boundaries freely, so the work per wave differs
// by at most one step whatever the context lengths.  A row block r (counted
// over the call) covered by waves w0..w1 leaves its piece from wave w in
// piece slot r + w (see BalancedSplit), and the merge recomputes w0 and w1
// from the same formula; a row block that one wave covers is written to the
// output directly.
template <typename T, typename KV, int D, int ROWS, bool DEBUG, bool UNIFORM>
__global__ __launch_bounds__(256) void decode_kernel(LaunchParams p, int row_blocks) {
  if (contract_broken(p)) return;
  constexpr int kWaves = 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (!p.balanced) {
    const int units = p.Hkv * row_blocks;
    const int idx = blockIdx.x * kWaves + wave;
    const int s = idx / units;
    const int u = idx - s * units;
    const int g = u / row_blocks;
    const int rb = u - g * row_blocks;
    const int b = blockIdx.y;
    if (s >= p.num_splits) return;
    const int ctx = p.cl[b];
    const int Lb = query_rows(p, b);
    if (!routed_here(p, Lb)) return;
    const int t0 = s * p.part_tokens;
    if (s > 0 && t0 >= ctx) return;  // never read by the merge
    const bool split = p.num_splits > 1;
    const ItemOut io{s, -1, 0, 0, 0};
    decode_item<T, KV, D, ROWS, DEBUG, UNIFORM>(p, b, g, rb, t0, split ? t0 + p.part_tokens : ctx,
                                                io, split, ctx, Lb, p.qsl ? p.qsl[b] : 0);
    return;
  }

  // ---- balanced schedule: prefix sums of the per-request step counts
  constexpr int kStep = decode_step_keys(D, (int)sizeof(KV));
  __shared__ long long s_R[kBalancedMaxBatch + 1];  // first step of request b
  __shared__ int s_ctx[kBalancedMaxBatch];
  __shared__ int s_pre[kBalancedMaxBatch];  // shared-prefix keys of request b (0: none)
  // query rows of request b and (packed rows) its first row: read once here
  // rather than by every piece's setup, where they would add a round trip
  __shared__ int s_rows[kBalancedMaxBatch], s_q0[kBalancedMaxBatch];
  __shared__ long long s_wsum[4];  // wave totals of the prologue's scans
  const int B = p.B;
  const int U = p.Hkv * row_blocks;
  const int tid = threadIdx.x;
  // per-thread serial sums over a contiguous slice, then a block scan
  const int per = (B + 255) / 256;
  const bool shared = p.grp_start != nullptr;
  if (shared) {
    // Shared prefixes: each non-empty group marks its first request, and the
    // first request past the groups is marked num_groups (no group); the
    // groups are consecutive ranges from request 0, so an inclusive max scan
    // of the marks over the requests names the group of every request.
    for (int b = tid; b < B; b += 256) s_pre[b] = -1;
    __syncthreads();
    for (int k = tid; k <= p.num_groups; k += 256) {
      const int first = p.grp_start[k];
      const bool mark = k == p.num_groups || first < p.grp_start[k + 1];  // distinct positions
      if (mark && first >= 0 && first < B) s_pre[first] = k;
    }
    __syncthreads();
    long long mark = -1;
    for (int k = 0; k < per; ++k) {
      const int b = tid * per + k;
      if (b < B) mark = max(mark, (long long)s_pre[b]);
    }
    long long grp;  // exclusive max scan of the marks
    block_scan(mark, -1ll, [](long long x, long long y) { return x > y ? x : y; }, s_wsum, &grp);
    for (int k = 0; k < per; ++k) {  // this thread's slice only: no other thread reads it
      const int b = tid * per + k;
      if (b < B) {
        grp = max(grp, (long long)s_pre[b]);
        s_pre[b] = grp >= 0 && grp < p.num_groups ? group_prefix_keys(p, (int)grp) : 0;
      }
    }
    __syncthreads();  // s_wsum is reused below
  } else {
    for (int b = tid; b < B; b += 256) s_pre[b] = 0;  // read after the scan's barriers
  }
  long long loc = 0;
  for (int k = 0; k < per; ++k) {
    const int b = tid * per + k;
    if (b < B) {
      // a request of another route counts as one without keys; a request of
      // a shared-prefix group walks only its keys past the prefix
      const int lb = query_rows(p, b);
      const int ctx = routed_here(p, lb) ? p.cl[b] : -1;
      s_ctx[b] = ctx;
      s_rows[b] = lb;
      s_q0[b] = p.qsl ? p.qsl[b] : 0;
      const int keys = ctx - (shared ? s_pre[b] : 0);
      const int n = keys > 0 ? (keys + kStep - 1) / kStep : 0;
      loc += (long long)U * (n > 0 ? n + kUnitSetupSteps : 0);
    }
  }
  long long run;  // exclusive sum scan of the step positions
  const long long total =
      block_scan(loc, 0ll, [](long long x, long long y) { return x + y; }, s_wsum, &run);
  for (int k = 0; k < per; ++k) {
    const int b = tid * per + k;
    if (b < B) {
      const int keys = s_ctx[b] - s_pre[b];
      const int n = keys > 0 ? (keys + kStep - 1) / kStep : 0;
      s_R[b] = run;
      run += (long long)U * (n > 0 ? n + kUnitSetupSteps : 0);
    }
  }
  if (tid == 255) s_R[B] = total;
  __syncthreads();

  // Values read from LDS are per-lane to the compiler; everything that shapes
  // the walk is made wave-uniform (scalar) so that loop bounds and buffer
  // descriptors stay in scalar registers.
  auto uni = [](int v) { return __builtin_amdgcn_readfirstlane(v); };
  auto uni64 = [](long long v) {
    const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)v);
    const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)((unsigned long long)v >> 32));
    return (long long)(((unsigned long long)hi << 32) | lo);
  };
  const long long Tot = uni64(s_R[B]);
  const long long units_all = (long long)B * U;
  const BalancedSplit bs = balanced_split(p.grid_waves, Tot, units_all, p.num_splits);
  const long long w = (long long)blockIdx.x * kWaves + wave;
  const int lane = threadIdx.x & 63;
  // A request without keys has no steps: wave (b mod grid waves) writes its
  // (zero) output rows (a request of another route, marked -1, is left alone;
  // so is one with keys past a shared prefix).
  {
    for (int b = (int)w; b < B; b += (int)gridDim.x * kWaves) {
      const int ctx = uni(s_ctx[b]);
      if (ctx < 0 || ctx - uni(s_pre[b]) > 0) continue;
      const size_t first = query_row(p, b, 0, 0) * D;
      const size_t row_elems = (size_t)p.Hq * (p.qsl ? query_rows(p, b) : p.L) * D;
      uint4 *dst = reinterpret_cast<uint4 *>(reinterpret_cast<T *>(p.out) + first);
      const size_t n16 = row_elems * sizeof(T) / 16;
      for (size_t i = lane; i < n16; i += 64) dst[i] = make_uint4(0, 0, 0, 0);
    }
  }

  // The steps of the run of wave v (positions [begin(v), begin(v + 1))),
  // piece by piece: a piece is the part of one row block inside the run.
  // Positions of the step order: each row block with keys is kUnitSetupSteps
  // setup positions (no work) followed by its n steps.
  auto run_segment = [&](long long v) {
    long long t = bs.begin(v);
    const long long e = bs.begin(v + 1);
    while (t < e) {
      int lo = 0, hi = B - 1;  // request: the largest b with s_R[b] <= t
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_R[mid] <= t) lo = mid; else hi = mid - 1;
      }
      const int b = uni(lo);
      const int ctx = uni(s_ctx[b]);
      const int pre = uni(s_pre[b]);  // keys below pre: the group's prefix state
      const long long n = (ctx - pre + kStep - 1) / kStep;  // > 0: request b holds position t
      const long long nu = n + kUnitSetupSteps;       // positions per row block
      const long long Rb = uni64(s_R[b]);
      const long long rel = t - Rb;
      const int u = (int)(rel / nu);
      const long long row0 = Rb + (long long)u * nu + kUnitSetupSteps;  // first step
      if (t < row0) {  // inside the setup positions: the row block starts at row0
        t = row0;
        continue;
      }
      const long long j0 = t - row0;
      const long long j1 = min(n, j0 + (e - t));
      const long long w0 = bs.wave_of(row0);
      const long long w1 = bs.wave_of(row0 + n - 1);
      const int g = u / row_blocks;
      const int rb = u - g * row_blocks;
      const int Lb = uni(s_rows[b]);
      const long long unit = (long long)b * U + u;  // row block over the call
      const ItemOut io{0, unit + v, unit + w0, (int)(w1 - w0 + 1), unit};
      // a row block with a prefix state always goes through the merge
      decode_item<T, KV, D, ROWS, DEBUG, UNIFORM>(p, b, g, rb, pre + (int)(j0 * kStep),
                                                  pre + (int)(j1 * kStep), io,
                                                  w1 > w0 || pre > 0, ctx, Lb, uni(s_q0[b]),
                                                  pre > 0);
      t += j1 - j0;
    }
  };

  if (w < bs.Wa) run_segment(w);
}

// Workgroups of `kernel` that fit on the current device at once, cached in
// `cached` (one array per kernel) per device.
template <typename K>
int resident_blocks(K kernel, int (&cached)[64]) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (cached[dev] == 0) {
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 256, 0) != hipSuccess ||
        per_cu < 1)
      per_cu = 1;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus < 1)
      cus = 256;
    cached[dev] = per_cu * cus;
  }
  return cached[dev];
}

// The kernel variant for `p` is chosen once, here; `Fn` either launches it
// or reports its balanced grid size.
template <typename T, typename KV, int D, int ROWS, bool DEBUG, bool UNIFORM>
struct Variant {
  static hipError_t launch(const LaunchParams &p, int row_blocks, hipStream_t stream) {
    auto kernel = decode_kernel<T, KV, D, ROWS, DEBUG, UNIFORM>;
    dim3 grid;
    if (p.balanced) {
      grid = dim3((unsigned)(p.grid_waves / 4), 1, 1);
    } else {
      const long per_request = ((long)p.Hkv * row_blocks * p.num_splits + 3) / 4;
      grid = dim3((unsigned)per_request, p.B, 1);
    }
    hipLaunchKernelGGL(kernel, grid, dim3(256), 0, stream, p, row_blocks);
    return hipGetLastError();
  }
  static int waves() {
    static int cached[64] = {0};
    return 4 * resident_blocks(decode_kernel<T, KV, D, ROWS, DEBUG, UNIFORM>, cached);
  }
};

template <typename T, typename KV, int D, int ROWS, typename Fn>
auto dispatch_mode(const LaunchParams &p, Fn &&fn) {
  // keys one page resolution covers (the page-uniform walk needs pages made
  // of whole resolutions): a step, or 16 keys for fp8 pages
  constexpr int kResKeys = sizeof(KV) == 1 ? 16 : decode_step_keys(D, (int)sizeof(KV));
  const bool uniform = p.ps % kResKeys == 0;
  const bool debug = p.dbg_trace != nullptr || p.dbg_visits != nullptr;
  if (debug)
    return uniform ? fn(Variant<T, KV, D, ROWS, true, true>())
                   : fn(Variant<T, KV, D, ROWS, true, false>());
  return uniform ? fn(Variant<T, KV, D, ROWS, false, true>())
                 : fn(Variant<T, KV, D, ROWS, false, false>());
}

template <typename X>
struct TypeTag {
  using type = X;
};

template <typename Fn>
auto dispatch(const LaunchParams &p, DType dt, Fn &&fn) {
  const int rows = decode_rows_per_block((p.Hq / p.Hkv) * p.L);
  auto by_rows = [&](auto t, auto kv, auto d) {
    using TT = typename decltype(t)::type;
    using KK = typename decltype(kv)::type;
    constexpr int DD = decltype(d)::value;
    switch (rows) {
      case 1: return dispatch_mode<TT, KK, DD, 1>(p, fn);
      case 2: return dispatch_mode<TT, KK, DD, 2>(p, fn);
      case 4: return dispatch_mode<TT, KK, DD, 4>(p, fn);
      default: return dispatch_mode<TT, KK, DD, 8>(p, fn);
    }
  };
  using F = TypeTag<float>;
  using H = TypeTag<uint16_t>;
  using E = TypeTag<uint8_t>;  // fp8 E4M3 codes
  using D64 = std::integral_constant<int, 64>;
  using D128 = std::integral_constant<int, 128>;
  if (dt == DType::F32) return p.D == 64 ? by_rows(F(), F(), D64()) : by_rows(F(), F(), D128());
  if (p.kv_fp8) return by_rows(H(), E(), D128());  // the host admits D = 128 only
  return p.D == 64 ? by_rows(H(), H(), D64()) : by_rows(H(), H(), D128());
}

}  // namespace

hipError_t launch_decode(const LaunchParams &p, DType dt, hipStream_t stream) {
  const int row_blocks =
      ((p.Hq / p.Hkv) * p.L + decode_rows_per_block((p.Hq / p.Hkv) * p.L) - 1) /
      decode_rows_per_block((p.Hq / p.Hkv) * p.L);
  return dispatch(p, dt, [&](auto v) { return decltype(v)::launch(p, row_blocks, stream); });
}

int decode_balanced_waves(const LaunchParams &p, DType dt) {
  return dispatch(p, dt, [](auto v) { return decltype(v)::waves(); });
}

}  // namespace pa
