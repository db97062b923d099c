// Paged decode kernel (vector ALU) for gfx950, with split-KV partitions.
//
// Schedule (tiny-llm "Week 3 Day 4", "Choose a Schedule for Each Query Shape"
// and "Checkpoint 2": parallelise short queries across the cached context,
// coalesce lanes over head elements, resolve a page id once per page, keep
// the query and the softmax state in registers, reduce with cross-lane
// operations; "Reading vLLM's PagedAttention Kernel" section 3.3: split long
// contexts into partitions that are merged afterwards):
//
//   grid  = (partition s, kv head g x row block, request b), 256 threads.
//   A workgroup owns the ROWS packed query rows (row rho -> position
//   rho / G, head g*G + rho % G) of one kv head, so each K/V byte of the
//   partition is read once for all of them.  Its 4 waves take interleaved
//   steps of STEP keys.  In a step every lane issues 16-byte loads: LPT
//   lanes cover one key's D elements and a wave load covers TPL keys, so the
//   loads of a page are fully coalesced.  Dot products are summed over the
//   LPT lanes with DPP; the (max, sum, output) state is kept per row in
//   registers and rescaled with exp2 (scores are in base-2 units).  At the end
//   the token groups and the waves are merged through LDS and the partition
//   state is written (normalised output + log-sum-exp), or the final output
//   when there is a single partition.
#include "pa_common.hpp"
#include "pa_internal.h"

namespace pa {
namespace {

using Vec = uint4;  // one 16-byte lane load

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

template <typename T, int D, int ROWS, bool DEBUG>
__global__ __launch_bounds__(256) void decode_kernel(LaunchParams p, int row_blocks) {
  constexpr int kElems = Elem<T>::kPerVec;
  constexpr int kLpt = D / kElems;      // lanes per key
  constexpr int kTpl = 64 / kLpt;       // keys per wave load
  constexpr int kLoads = 4;             // loads in flight per step (each of K and V)
  constexpr int kStep = kTpl * kLoads;  // keys per wave step
  constexpr int kWaves = 4;
  static_assert(kLpt * kElems == D && kTpl * kLpt == 64, "layout");

  const int s = blockIdx.x;
  const int g = blockIdx.y / row_blocks;
  const int rb = blockIdx.y - g * row_blocks;
  const int b = blockIdx.z;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int c = lane % kLpt;            // element chunk of this lane
  const int kl = lane / kLpt;           // key of this lane within a load

  const int G = p.Hq / p.Hkv;
  const int ctx = p.cl[b];
  const int Lb = p.ql ? p.ql[b] : p.L;
  const int t0 = s * p.part_tokens;
  const bool split = p.num_splits > 1;
  if (split && t0 >= ctx) return;  // empty partition: the merge never reads it

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
    qrow[r] = ((size_t)(b * p.Hq + h) * p.L + i);
    kmax = max(kmax, hi[r]);
    if (valid[r]) kmin = min(kmin, hi[r]);
  }
  const int t1 = split ? min(t0 + p.part_tokens, kmax) : kmax;
  // last packed row of the request decides which row block counts visits
  const bool counts = DEBUG && ((Lb * G - 1) / ROWS == rb) && Lb > 0;

  Vec qv[ROWS];
  const T *qbase = reinterpret_cast<const T *>(p.q);
#pragma unroll
  for (int r = 0; r < ROWS; ++r) {
    qv[r] = valid[r] ? *reinterpret_cast<const Vec *>(qbase + qrow[r] * D + c * kElems)
                     : make_uint4(0, 0, 0, 0);
  }

  float m[ROWS], l[ROWS], acc[ROWS][kElems];
#pragma unroll
  for (int r = 0; r < ROWS; ++r) {
    m[r] = kNegInf;
    l[r] = 0.f;
#pragma unroll
    for (int e = 0; e < kElems; ++e) acc[r][e] = 0.f;
  }

  const T *kp = reinterpret_cast<const T *>(p.kp);
  const T *vp = reinterpret_cast<const T *>(p.vp);
  const int32_t *bt = p.bt + (size_t)b * p.max_pages;
  const int ps = p.ps;
  const bool uniform_page = (ps % kStep) == 0;
  const int nsteps = t1 > t0 ? (t1 - t0 + kStep - 1) / kStep : 0;
  const int tmin = min(t1, kmin);  // keys below this are visible to every valid row

  auto lane_offset = [&](int base, int n, int &page, int &slot) -> size_t {
    int j = base + n * kTpl + kl;
    if (uniform_page) {
      const int lp = base / ps;
      page = __builtin_amdgcn_readfirstlane(bt[lp]);
      slot = base - lp * ps + n * kTpl + kl;
    } else {
      j = min(j, t1 - 1);  // keys past the end reuse a valid address; masked below
      const int lp = j / ps;
      page = bt[lp];
      slot = j - lp * ps;
    }
    return ((size_t)page * p.Hkv + g) * ps * D + (size_t)slot * D + c * kElems;
  };

  auto load_step = [&](int step, Vec (&kv)[kLoads], Vec (&vv)[kLoads]) {
    const int base = t0 + step * kStep;
#pragma unroll
    for (int n = 0; n < kLoads; ++n) {
      int page, slot;
      const size_t off = lane_offset(base, n, page, slot);
      kv[n] = *reinterpret_cast<const Vec *>(kp + off);
      vv[n] = *reinterpret_cast<const Vec *>(vp + off);
      if constexpr (DEBUG) {
        const int j = base + n * kTpl + kl;
        if (counts && c == 0 && j < t1) {
          if (g == 0) {
            p.dbg_trace[((size_t)b * p.max_pages * ps + j) * 2 + 0] = page;
            p.dbg_trace[((size_t)b * p.max_pages * ps + j) * 2 + 1] = slot;
          }
          atomicAdd(&p.dbg_visits[((size_t)b * p.Hkv + g) * p.max_pages * ps + j], 1);
        }
      }
    }
  };

  auto fold_step = [&](int step, const Vec (&kv)[kLoads], const Vec (&vv)[kLoads]) {
    const int base = t0 + step * kStep;
    const bool tail = base + kStep > tmin;
    float sc[kLoads][ROWS];
#pragma unroll
    for (int n = 0; n < kLoads; ++n) {
#pragma unroll
      for (int r = 0; r < ROWS; ++r) {
        sc[n][r] = group_sum<kLpt>(lane_dot<T>(qv[r], kv[n])) * p.scale_log2;
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
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
      float mx = sc[0][r];
#pragma unroll
      for (int n = 1; n < kLoads; ++n) mx = fmaxf(mx, sc[n][r]);
      mx = stride_max<kLpt>(mx);
      const float mnew = fmaxf(m[r], mx);
      const bool none = mnew == kNegInf;
      const float alpha = none ? 1.f : fast_exp2(m[r] - mnew);
      m[r] = mnew;
      l[r] *= alpha;
#pragma unroll
      for (int e = 0; e < kElems; ++e) acc[r][e] *= alpha;
#pragma unroll
      for (int n = 0; n < kLoads; ++n) {
        const float pr = none ? 0.f : fast_exp2(sc[n][r] - mnew);
        sc[n][r] = pr;
        l[r] += pr;
      }
    }
#pragma unroll
    for (int n = 0; n < kLoads; ++n) {
      float vf[kElems];
      widen<T>(vv[n], vf);
      if (tail && base + n * kTpl + kl >= t1) {
        // stale slots past the context may hold anything, NaN included
#pragma unroll
        for (int e = 0; e < kElems; ++e) vf[e] = 0.f;
      }
#pragma unroll
      for (int r = 0; r < ROWS; ++r) {
#pragma unroll
        for (int e = 0; e < kElems; ++e) acc[r][e] = fmaf(sc[n][r], vf[e], acc[r][e]);
      }
    }
  };

  // ---- main walk: wave w takes steps w, w + 4, ...; the next step's loads
  // are issued before the current step is folded.
  if (wave < nsteps) {
    Vec kc[kLoads], vc[kLoads];
    load_step(wave, kc, vc);
    for (int step = wave; step < nsteps; step += kWaves) {
      Vec kn[kLoads], vn[kLoads];
      const bool more = step + kWaves < nsteps;
      if (more) load_step(step + kWaves, kn, vn);
      fold_step(step, kc, vc);
      if (more) {
#pragma unroll
        for (int n = 0; n < kLoads; ++n) { kc[n] = kn[n]; vc[n] = vn[n]; }
      }
    }
  }

  // ---- merge token groups within the wave, then the waves through LDS
  __shared__ float sm_acc[kWaves][ROWS][D];
  __shared__ float sm_m[kWaves][ROWS];
  __shared__ float sm_l[kWaves][ROWS];
#pragma unroll
  for (int r = 0; r < ROWS; ++r) {
    const float lt = stride_sum<kLpt>(l[r]);
#pragma unroll
    for (int e = 0; e < kElems; ++e) acc[r][e] = stride_sum<kLpt>(acc[r][e]);
    if (lane < kLpt) {
#pragma unroll
      for (int e = 0; e < kElems; ++e) sm_acc[wave][r][c * kElems + e] = acc[r][e];
    }
    if (lane == 0) {
      sm_m[wave][r] = m[r];
      sm_l[wave][r] = lt;
    }
  }
  __syncthreads();

  T *out = reinterpret_cast<T *>(p.out);
  for (int t = threadIdx.x; t < ROWS * D; t += 256) {
    const int r = t / D, d = t - r * D;
    const int rho = rb * ROWS + r;
    if (rho >= G * p.L) continue;
    const int i = rho / G;
    const int h = g * G + (rho - i * G);
    const size_t row = ((size_t)(b * p.Hq + h) * p.L + i);
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm_m[w][r]);
    float o = 0.f, lse = kNegInf;
    if (valid[r] && M != kNegInf) {
      float wsum = 0.f, osum = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float f = fast_exp2(sm_m[w][r] - M);
        wsum += f * sm_l[w][r];
        osum += f * sm_acc[w][r][d];
      }
      o = osum / wsum;
      lse = (M + __log2f(wsum)) * kLn2;
    }
    if (split) {
      if (!valid[r]) continue;  // the merge writes padding rows itself
      p.ws_o[(row * p.num_splits + s) * D + d] = o;
      if (d == 0) p.ws_lse[row * p.num_splits + s] = lse;
    } else {
      if constexpr (sizeof(T) == 4) {
        out[row * D + d] = o;
      } else {
        out[row * D + d] = (uint16_t)f32_to_bf16(o);
      }
    }
  }
}

template <typename T, int D, int ROWS>
hipError_t launch_typed(const LaunchParams &p, hipStream_t stream) {
  const int G = p.Hq / p.Hkv;
  const int row_blocks = (G * p.L + ROWS - 1) / ROWS;
  dim3 grid(p.num_splits, p.Hkv * row_blocks, p.B);
  const bool debug = p.dbg_trace != nullptr || p.dbg_visits != nullptr;
  if (debug) {
    hipLaunchKernelGGL((decode_kernel<T, D, ROWS, true>), grid, dim3(256), 0, stream, p, row_blocks);
  } else {
    hipLaunchKernelGGL((decode_kernel<T, D, ROWS, false>), grid, dim3(256), 0, stream, p, row_blocks);
  }
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_rows(const LaunchParams &p, hipStream_t stream) {
  switch (decode_rows_per_block((p.Hq / p.Hkv) * p.L)) {
    case 1: return launch_typed<T, D, 1>(p, stream);
    case 2: return launch_typed<T, D, 2>(p, stream);
    case 4: return launch_typed<T, D, 4>(p, stream);
    default: return launch_typed<T, D, 8>(p, stream);
  }
}

}  // namespace

hipError_t launch_decode(const LaunchParams &p, DType dt, hipStream_t stream) {
  if (dt == DType::F32) {
    return p.D == 64 ? launch_rows<float, 64>(p, stream) : launch_rows<float, 128>(p, stream);
  }
  return p.D == 64 ? launch_rows<uint16_t, 64>(p, stream) : launch_rows<uint16_t, 128>(p, stream);
}

}  // namespace pa
