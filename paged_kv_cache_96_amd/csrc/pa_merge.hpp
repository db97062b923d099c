// Log-sum-exp merge of split-KV partial states for one query row ("Reading
// vLLM's PagedAttention Kernel", section 3.3: partial results computed in
// parallel are combined afterwards):
//   M = max_s lse_s,  w_s = exp(lse_s - M),  out = sum_s w_s o_s / sum_s w_s,
// zeros when no state saw a key (every lse_s = -inf).  Used by the merge
// kernel and by the decode kernel's fused merge.  The states are read with
// system-scope loads, which bypass the (per-XCD, non-coherent) L2: a merging
// wave may read states that waves on other XCDs wrote moments before.
#pragma once

#include "pa_common.hpp"
#include "pa_internal.h"

namespace pa {

// Cache-policy bits of buffer instructions on gfx94x/gfx950: sc0 | sc1
// (system scope: stores write through to memory, loads miss every cache).
constexpr int kSysScope = 1 | 16;

// How the fused merges (decode and prefill) publish piece states across
// XCDs.  Each XCD has its own L2, not coherent with the others for ordinary
// device memory.  The agent-scope release / acquire fences the compiler emits
// for this target write back and invalidate a whole L2; measured on MI355X
// they slowed the 64-request decode from 113 to 165 us and the chunked
// prefill from 50 to 96 us.  The merges order the accesses that matter one
// by one instead:
//   1. every piece-state store carries sc0 | sc1: written through every cache
//      to memory;
//   2. s_waitcnt vmcnt(0) waits until those stores are acknowledged, i.e.
//      have reached memory;
//   3. the arrival counter is an agent-scope atomic, performed at memory;
//   4. the wave that completes the count reads the states with sc0 | sc1
//      loads, which miss every cache, after a compiler barrier that keeps
//      them below the atomic.
// The guarantee rests on the gfx950 meaning of the sc0 / sc1 bits and of
// the store acknowledgement that vmcnt counts; the library is built for that
// target only, and this check keeps it so.
#if defined(__HIP_DEVICE_COMPILE__) && !defined(__gfx950__)
#error "the fused merges rely on gfx950 cache-policy bits; build for gfx950"
#endif

// Natural-log -> base-2 factor for the exponent weights.
constexpr float kMergeLog2e = 1.44269504088896340736f;

// Merge n states of one row.  State s lives at element offset s * stride of
// `lse` and at row (s * stride) of `po` (rows of D floats).  Every lane of
// the wave takes part; lane l writes output elements e * 64 + l.
template <typename T, int D>
__device__ __forceinline__ void merge_row(const float *lse, const float *po, int stride, int n,
                                          T *out_row) {
  constexpr int kPer = D / 64;
  const int lane = threadIdx.x & 63;
  const __amdgpu_buffer_rsrc_t rl = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float *>(lse), (short)0, 0x7fffffff, kBufferRsrcWord3);
  const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float *>(po), (short)0, 0x7fffffff, kBufferRsrcWord3);
  // the loads return raw 32-bit words: reinterpret, never convert
  auto load_f32 = [](__amdgpu_buffer_rsrc_t r, int byte_off) {
    return __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, kSysScope));
  };
  float M = kNegInf;
  for (int s = lane; s < n; s += 64) M = fmaxf(M, load_f32(rl, s * stride * 4));
  M = group_max<64>(M);
  float o[kPer];
#pragma unroll
  for (int e = 0; e < kPer; ++e) o[e] = 0.f;
  if (M != kNegInf) {
    float wsum = 0.f;
    for (int s = 0; s < n; ++s) {
      const float ls = load_f32(rl, s * stride * 4);
      const float w = fast_exp2((ls - M) * kMergeLog2e);
      wsum += w;
#pragma unroll
      for (int e = 0; e < kPer; ++e) {
        const float v = load_f32(ro, (s * stride * D + e * 64 + lane) * 4);
        o[e] = fmaf(w, v, o[e]);
      }
    }
    const float inv = 1.f / wsum;
#pragma unroll
    for (int e = 0; e < kPer; ++e) o[e] *= inv;
  }
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    if constexpr (sizeof(T) == 4) {
      out_row[e * 64 + lane] = o[e];
    } else {
      out_row[e * 64 + lane] = (uint16_t)f32_to_bf16(o[e]);
    }
  }
}

}  // namespace pa

namespace pa {

// Merge the n pieces of a block of R rows in one pass, all rows at once:
// 64 / R lanes per row, each owning D * R / 64 consecutive elements.  Piece s
// of row r has its state at lse[s * R + r] and po[(s * R + r) * D ...]; rows
// with valid[r] false get zeros.  A running (max, sum, acc) keeps every load
// independent of the previous piece's arithmetic, and the loop body has no
// branch (an all-empty prefix is carried by selects), so the unrolled loads
// of up to 16 pieces are in flight together: the states are read past the
// caches, and a row block split into many pieces (a small batch over long
// contexts) would otherwise pay one memory round trip per piece.
// With pre_lse (shared-prefix decode) every valid row first folds its
// prefix states: pre_n[row] of them, state s at pre_lse[row * kPrefixPieces
// + s] and pre_o[(row * kPrefixPieces + s) * D ...] by the row's output
// index, which an earlier launch on the stream wrote (ordinary loads see
// it).
template <typename T, int D, int R>
__device__ __forceinline__ void merge_block(const float *lse, const float *po, int n,
                                            const bool (&valid)[R], const size_t (&qrow)[R],
                                            int rows_in_range, T *out,
                                            const float *pre_lse = nullptr,
                                            const float *pre_o = nullptr,
                                            const int32_t *pre_n = nullptr) {
  constexpr int kLanes = 64 / R;       // lanes per row
  constexpr int kE = D / kLanes;       // elements per lane
  static_assert(kLanes * R == 64 && kE * kLanes == D && kE % 4 == 0 || kE < 4, "layout");
  const int lane = threadIdx.x & 63;
  const int r = lane / kLanes;
  const int e0 = (lane % kLanes) * kE;
  bool ok = false;
  size_t row = 0;
#pragma unroll
  for (int i = 0; i < R; ++i)
    if (i == r) {
      ok = valid[i] && i < rows_in_range;
      row = qrow[i];
    }
  const int cnt = ok ? n : 0;
  const __amdgpu_buffer_rsrc_t rl = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float *>(lse), (short)0, 0x7fffffff, kBufferRsrcWord3);
  const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float *>(po), (short)0, 0x7fffffff, kBufferRsrcWord3);
  // state (m, l, acc): output acc / l, log-sum-exp m + ln l
  float m = kNegInf, l = 0.f, acc[kE];
#pragma unroll
  for (int e = 0; e < kE; ++e) acc[e] = 0.f;
  // fold one state (log-sum-exp ls, normalised output v)
  auto fold = [&](float ls, const float (&v)[kE]) {
    const float mn = fmaxf(m, ls);
    const bool none = mn == kNegInf;  // nothing seen yet: the state stays (-inf, 0, 0)
    const float a = none ? 0.f : fast_exp2((m - mn) * kMergeLog2e);  // m = -inf -> 0
    const float w = none ? 0.f : fast_exp2((ls - mn) * kMergeLog2e);
    m = mn;
    l = fmaf(l, a, w);
#pragma unroll
    for (int e = 0; e < kE; ++e) acc[e] = none ? 0.f : fmaf(acc[e], a, w * v[e]);
  };
  if (pre_lse != nullptr && ok) {
    // batches of kBatch slots, all loaded at once (every slot of the row
    // lies in the buffer; slots past the count are loaded but not folded)
    constexpr int kBatch = kE <= 4 ? 16 : kE <= 8 ? 8 : 4;
    static_assert(kPrefixPieces % kBatch == 0, "batches");
    const int npre = min(pre_n[row], kPrefixPieces);  // the same for every row of the block
    const float *pl = pre_lse + row * kPrefixPieces;
    const float *pv = pre_o + row * kPrefixPieces * D + e0;
    for (int s0 = 0; s0 < npre; s0 += kBatch) {
      float ls[kBatch], v[kBatch][kE];
#pragma unroll
      for (int k = 0; k < kBatch; ++k) {
        ls[k] = pl[s0 + k];
#pragma unroll
        for (int e = 0; e < kE; ++e) v[k][e] = pv[(s0 + k) * D + e];
      }
#pragma unroll
      for (int k = 0; k < kBatch; ++k)
        if (s0 + k < npre) fold(ls[k], v[k]);
    }
  }
#pragma unroll 16
  for (int s = 0; s < cnt; ++s) {
    const float ls = __uint_as_float(
        (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rl, (s * R + r) * 4, 0, kSysScope));
    float v[kE];
    const int base = ((s * R + r) * D + e0) * 4;
    if constexpr (kE >= 4) {
#pragma unroll
      for (int e = 0; e < kE; e += 4) {
        const u32x4_t q = __builtin_amdgcn_raw_buffer_load_b128(ro, base + e * 4, 0, kSysScope);
        v[e] = __uint_as_float(q[0]);
        v[e + 1] = __uint_as_float(q[1]);
        v[e + 2] = __uint_as_float(q[2]);
        v[e + 3] = __uint_as_float(q[3]);
      }
    } else {
#pragma unroll
      for (int e = 0; e < kE; ++e)
        v[e] = __uint_as_float(
            (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(ro, base + e * 4, 0, kSysScope));
    }
    fold(ls, v);
  }
  if (r >= rows_in_range) return;
  const float inv = l > 0.f ? 1.f / l : 0.f;
  T *dst = out + row * D + e0;
#pragma unroll
  for (int e = 0; e < kE; ++e) {
    if constexpr (sizeof(T) == 4) {
      dst[e] = acc[e] * inv;
    } else {
      dst[e] = (uint16_t)f32_to_bf16(acc[e] * inv);
    }
  }
}

}  // namespace pa
