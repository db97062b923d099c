// bf16 paged prefill kernel on gfx950 matrix cores (pages of bf16 values or
// of fp8 E4M3 codes with per-tensor scales).
//
// Work: one workgroup (4 waves) owns BM = 128 * RB packed query rows of one
// (request b, kv head g); packed row rho is position rho / G of head
// g*G + rho % G, so the G heads that share a kv head share every K/V tile and
// the rows of a tile sit at nearly the same causal position.  A wave owns RB
// blocks of 32 rows: every K and V operand it reads from LDS feeds RB matrix
// instructions (the launcher uses RB = 1; see launch_d).  Keys are walked
// in tiles of BN = 32 (LDS loads, below) or 64 keys (tiny-llm "Week 3 Day
// 4", "Task 2": resolve every K/V tile through the block table, fold it in
// with the online softmax).
//
// Per key tile:
//   1. staging, with two LDS buffers and one barrier per tile.  When
//      page_size is a multiple of 8, each wave's 8-key run of a tile lies in
//      one page: its block-table entry is a scalar load (SGPR) and the run
//      is read with buffer loads from that page at per-lane offsets fixed
//      for the whole walk, so staging costs no per-lane address arithmetic.
//      The loads write LDS directly (kStageDma; kStageDmaRun for pools of
//      2 GiB and more, with one buffer resource per run): 32-key tiles,
//      wave w loads keys 8w .. 8w + 7 of the next
//      tile into the other buffer once the current tile's scores are
//      computed; no staging registers and no LDS stores, so a workgroup
//      needs 33 KiB of LDS and fits three waves per SIMD (the launch
//      bounds ask for three workgroups per compute unit); the tile layout
//      (dma_pos) keeps the operand reads conflict-free.  fp8 codes take the
//      same loads into a tile of half the bytes (fp8_pos), and each operand
//      read widens its 8 codes to bf16 (the transposed V read is the 8-bit
//      one; the key rows of the score product are permuted so that a lane's
//      PV keys are consecutive, fp8_key_perm); bf16 rows of D = 64 are 128
//      bytes as well and take that layout.  Page sizes that are not a
//      multiple of 8 take the same loads with each row's page resolved per
//      lane (kStageDmaLanes).  Register staging remains for such page sizes
//      on pools of 2 GiB and more: every thread loads the next tile into
//      registers and stores the set loaded one tile earlier to the other
//      LDS buffer;
//   2. S^T = K . Q^T with v_mfma_f32_32x32x16_bf16: K from LDS is the A
//      operand, Q (kept in registers for the whole walk) the B operand.  The
//      result gives every lane the scores of ONE query row (lane % 32) against
//      16 of the tile's keys; the other 16 sit in lane ^ 32;
//   3. softmax in registers (row max over the lane pair with a permlane32
//      swap, exp2 of pre-scaled scores, fp32 row sums), P rounded to bf16
//      once.  The weights of a row are taken relative to a reference max
//      fixed by the row's first key block (key 0 is visible to every row),
//      so O is never rescaled inside the walk and stays in accumulation
//      registers that only the matrix instructions touch.  Softmax does not
//      depend on the reference; bf16 and fp32 hold weights up to 2^16 with
//      the same relative precision as weights <= 1.  The true running max
//      is tracked, and if any row of the workgroup exceeds its reference by
//      more than 2^16 the workgroup walks its keys again with the exact max
//      as reference (weights <= 1), which keeps every input finite;
//   4. O^T += V^T . P^T with the same MFMA: P^T comes straight from the
//      lane's own registers (B operand); V^T (A operand) is read from the
//      natural [key][d] LDS tile with ds_read_b64_tr_b16, which hands each
//      lane four consecutive keys of one head dimension.
// Keys past a row's causal limit are masked on the diagonal tiles only, and
// tiles past the last row's limit are never loaded.
//
// Key split (with a workspace): a tile whose key range is much longer than
// the average work of a workgroup slot would bound the whole call (a long
// prefix in one request of the batch), so its keys are cut into pieces of
// at most P keys, each walked by its own workgroup, and the pieces are
// merged with the log-sum-exp rule of split-KV decoding ("Reading vLLM's
// PagedAttention Kernel", section 3.3).  Every workgroup derives the same
// plan from the context lengths (P = total work / (0.4 x workspace slots),
// at least kMinPieceKeys, a multiple of BN) and finds its piece by its
// index in the dispatch order, longest pieces first (see find_piece).  A split
// piece writes its state (unnormalised O, reference max and row sums) to
// its slot and counts its arrival on the tile's counter; the last piece to
// arrive reads them all back, merges them in piece order (so the result
// does not depend on the order of arrival) and writes the output.  No
// workgroup waits for another.
//
// Prefix launch of a shared-prefix decode (p.prefix_pass): one request per
// group of requests that share their first pages, holding the query rows
// of all the members over the shared keys; its tiles are cut into at most
// kPrefixPieces pieces, and each piece writes its own state of every member
// row (normalised output and log-sum-exp) for the decode kernel's merge,
// so nothing is merged here.
#include <type_traits>

#include "pa_common.hpp"
#include "pa_internal.h"
#include "pa_merge.hpp"

namespace pa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

constexpr int kBN = 64;    // keys per tile
constexpr float kMinM = -1.0e30f;  // reference sentinel: exp2(-inf - kMinM) = 0
constexpr float kRefSlack = 16.0f; // largest row max above the reference (log2) a walk accepts
// s_waitcnt immediate (gfx9 encoding): vmcnt <= 8 (the eight loads of one
// staging set may stay in flight), expcnt and lgkmcnt not waited for.
constexpr int kWaitVmcntOlderThan8 = 8 | (0x7 << 4) | (0xF << 8);
// Key split: shortest piece (the prefix launch of a shared-prefix decode:
// shorter, as its pieces are never merged here).
constexpr int kMinPieceKeys = 4 * kBN;
constexpr int kMinPrefixPieceKeys = 2 * kBN;

template <int D>
struct Tile {
  static constexpr int kKStride = D + 8;               // shorts per K row (pad 16 B)
  static constexpr int kVStride = D == 128 ? 160 : 96;  // shorts per V row (320 B / 192 B)
  static constexpr int kKBytes = kBN * kKStride * 2;
  static constexpr int kVBytes = kBN * kVStride * 2;
  static constexpr int kChunks = D / 8;                // 16-byte chunks per row
  static constexpr int kKeysPerRound = 256 / kChunks;
  static constexpr int kRounds = kBN / kKeysPerRound;
  static constexpr int kKSteps = D / 16;               // MFMA k-steps of QK^T
  static constexpr int kMBlocks = D / 32;              // 32-row blocks of O^T
};

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// Eight E4M3 codes (two words, element 0 in the low byte) as eight bf16
// values: every E4M3 value is a bf16 value, and the hardware converter of
// two codes to a bf16 pair (scale 1) gives it exactly.
__device__ __forceinline__ uint4 fp8x8_to_bf16x8(uint32_t w0, uint32_t w1) {
  auto lo = [](uint32_t w) {  // bytes 0, 1
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
  };
  auto hi = [](uint32_t w) {  // bytes 2, 3
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
  };
  return make_uint4(lo(w0), hi(w0), lo(w1), hi(w1));
}


// max(a, b, c) in one instruction, without the operand quieting that
// fmaxf adds (the scores are finite or -inf).
__device__ __forceinline__ float max3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
constexpr uint32_t kBf16OnePair = 0x3f803f80u;  // bf16 (1, 1)

// Max of a value held by lane l and lane l ^ 32.
__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return max3(__uint_as_float(r[0]), __uint_as_float(r[1]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP: row shifts
// within each 16-lane row, then the row totals broadcast to the later rows.
// Lanes whose source lies outside the row read 0.
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15 -> rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31 -> rows 2, 3
  return x;
}
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_add(float v) {
  return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROWS, 0xF, false));
}
__device__ __forceinline__ float wave_incl_scan_f(float x) {
  x = dpp_add<0x111, 0xF>(x);
  x = dpp_add<0x112, 0xF>(x);
  x = dpp_add<0x114, 0xF>(x);
  x = dpp_add<0x118, 0xF>(x);
  x = dpp_add<0x142, 0xA>(x);
  x = dpp_add<0x143, 0xC>(x);
  return x;
}

// Requests of a launch.  The prefix launch of a shared-prefix decode
// (p.prefix_pass) runs one request per group: request b holds the query rows
// of the group's members, p.Lm per member (member-major), over the group's
// shared prefix keys, without a mask (every member row sees its whole
// prefix).
__device__ __forceinline__ int launch_ctx(const LaunchParams &p, int b) {
  return p.prefix_pass ? group_prefix_keys(p, b) : p.cl[b];
}
__device__ __forceinline__ int launch_rows(const LaunchParams &p, int b) {
  return p.prefix_pass ? (p.grp_start[b + 1] - p.grp_start[b]) * p.Lm : query_rows(p, b);
}
// Query/output row index of row i < launch_rows(p, b) of head h; `exists`
// is false for a member's rows past its own query rows (prefix launch).
__device__ __forceinline__ size_t launch_row(const LaunchParams &p, int b, int h, int i,
                                             bool &exists) {
  exists = true;
  if (!p.prefix_pass) return query_row(p, b, h, i);
  const int j = i / p.Lm;
  const int pos = i - j * p.Lm;
  const int m = p.grp_start[b] + j;  // the member request
  if (p.qsl) {
    exists = pos < p.qsl[m + 1] - p.qsl[m];
    return (size_t)(p.qsl[m] + pos) * p.Hq + h;
  }
  exists = pos < (p.ql ? p.ql[m] : p.Lm);
  return ((size_t)m * p.Hq + h) * p.Lm + pos;
}

// The piece of the key split that workgroup blockIdx.x walks.
struct Piece {
  int tile, g, b;
  int k0, k1;  // keys [k0, k1) of the tile
  int np;      // pieces of the tile (1: not split)
  int sp;      // this piece
  int slot;    // first workspace slot of the tile's pieces (np > 1)
  int found;
};

// x / d for 0 <= x < 2^31, 0 < d: float estimate, then exact corrections
// (one step each way when x < 2^24).
__device__ __forceinline__ int div_small(int x, int d, float rcp) {
  long long q = (long long)((float)x * rcp);
  while (q * d > x) --q;
  while ((q + 1) * d <= x) ++q;
  return (int)q;
}

// Every workgroup computes the same plan (see the header).  Pairs (request,
// tile) are numbered by request, then tile from the last.  Total work W =
// H_kv * sum of the pairs' keys (in BN blocks); the work target of a piece
// is W / (0.4 S) (S workspace slots; measured best between W / (0.5 S) and
// W / (0.25 S)), and piece lengths are at most P = max(kMinPieceKeys,
// target) rounded up to BN; a pair with k > P keys splits into as equal
// pieces as the BN grid allows.  Dispatch order: longest pieces first, in
// four classes of piece length (>= 3P/4, >= P/2, >= P/4, shorter), each
// class in pair order; within a pair, kv head then piece.  Split pairs take
// workspace slots in pair order.  All 256 threads take part: each owns a
// contiguous slice of pairs, per-thread counts are scanned within waves
// (DPP) and across the four waves (LDS), and the thread whose slice holds
// this workgroup's piece publishes it in s_pc.  Pairs with no row to write
// (packed rows: a tile past the request's rows, or a request of the other
// route) form a fifth class after the four, so every piece with work has a
// lower index than every piece without, and a grid sized for the pairs that
// can have rows covers them all.  s_ctx, s_ql, s_len and s_keys:
// kSplitMaxPairs ints each, s_red 32 ints of scratch; the block
// synchronises before returning (the tables live in the staging buffers).
__device__ void find_piece(const LaunchParams &p, int nt, int *s_ctx, int *s_ql, int *s_len,
                           int *s_keys, int *s_red, Piece *s_pc, Piece &pc) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int G = p.Hq / p.Hkv;
  for (int b = tid; b < p.B; b += 256) {
    s_ctx[b] = launch_ctx(p, b);
    // a request of another route has no rows here (no keys, one empty piece)
    const int lb = launch_rows(p, b);
    s_ql[b] = routed_here(p, lb) ? lb : 0;
  }
  if (tid == 0) s_pc->found = 0;
  __syncthreads();
  const int NP = p.B * nt;
  const int per = (NP + 255) / 256;
  const int q0 = min(NP, tid * per), q1 = min(NP, q0 + per);
  const float rcpG = 1.0f / (float)G;
  // keys of this thread's pairs (request and tile stepped along the slice)
  int w = 0;  // in BN blocks (below 2^29)
  if (q0 < q1) {
    int b = q0 / nt;
    int t = nt - 1 - (q0 - b * nt);
    int ctx = s_ctx[b], Lb = s_ql[b];
    for (int q = q0; q < q1; ++q) {
      const int rho0 = t * 128;
      const int last = min(rho0 + 128, G * Lb) - 1;
      const int k = last < rho0 ? 0 : (p.causal ? ctx - Lb + div_small(last, G, rcpG) + 1 : ctx);
      // -1: a tile with no row to write (packed rows and the prefix launch
      // write only rows that exist; padded rows past query_lens are zeroed)
      s_keys[q] = (last < rho0 && (p.qsl || p.prefix_pass)) ? -1 : k;
      w += (k + kBN - 1) / kBN;
      if (--t < 0 && q + 1 < q1) {
        t = nt - 1;
        ++b;
        ctx = s_ctx[b];
        Lb = s_ql[b];
      }
    }
  }
  // total in fp32, summed in one fixed order (every workgroup gets the same
  // value; P only needs to be the same everywhere and about right)
  float *s_redf = reinterpret_cast<float *>(s_red + 24);
  {
    const float ws = __shfl(wave_incl_scan_f((float)w), 63, 64);
    if (lane == 0) s_redf[wave] = ws;
  }
  __syncthreads();
  const float work = ((s_redf[0] + s_redf[1]) + (s_redf[2] + s_redf[3])) * (float)p.Hkv;
  const float target = 0.4f * (float)max(2, p.num_splits);
  const float blocks = fminf(ceilf(work / target), (float)(1 << 24));  // P / BN
  const int P = max(p.prefix_pass ? kMinPrefixPieceKeys : kMinPieceKeys, (int)blocks * kBN);
  auto npieces = [&](int k, int len) { return k > len ? (k + len - 1) / len : 1; };
  auto cls = [&](int len) {
    return 4 * (long long)len >= 3LL * P ? 0 : 2 * (long long)len >= P ? 1
           : 4 * (long long)len >= P ? 2 : 3;
  };
  // piece class of pair q: four by length, then the pairs with no row
  auto pair_cls = [&](int q, int len) { return s_keys[q] < 0 ? 4 : cls(len); };
  int cnt[6] = {0, 0, 0, 0, 0, 0};  // widths of the five classes, split slots
  for (int q = q0; q < q1; ++q) {
    const int k = max(s_keys[q], 0);
    int len = k;
    if (k > P) {
      // the prefix launch cuts a tile into kPrefixPieces pieces at most
      const int n0 = min((k + P - 1) / P, p.prefix_pass ? kPrefixPieces : k);
      len = ((k + n0 - 1) / n0 + kBN - 1) / kBN * kBN;
    }
    s_len[q] = len;
    const int n = npieces(k, len);
    const int c = pair_cls(q, len);
    const int wdt = p.Hkv * n;
    cnt[0] += c == 0 ? wdt : 0;
    cnt[1] += c == 1 ? wdt : 0;
    cnt[2] += c == 2 ? wdt : 0;
    cnt[3] += c == 3 ? wdt : 0;
    cnt[4] += c == 4 ? wdt : 0;
    cnt[5] += n > 1 ? wdt : 0;
  }
  // exclusive prefix of each count over the block, and the class totals
  int ex[6];
#pragma unroll
  for (int v = 0; v < 6; ++v) {
    const int inc = wave_incl_scan(cnt[v]);
    ex[v] = inc - cnt[v];
    if (lane == 63) s_red[v * 4 + wave] = inc;
  }
  __syncthreads();
  int off[6];
  off[0] = 0;
#pragma unroll
  for (int v = 0; v < 6; ++v) {
    int before = 0, tot = 0;
#pragma unroll
    for (int w2 = 0; w2 < 4; ++w2) {
      const int x = s_red[v * 4 + w2];
      before += w2 < wave ? x : 0;
      tot += x;
    }
    ex[v] += before;
    if (v < 5) off[v + 1] = off[v] + tot;
  }
  const int i = blockIdx.x;
  int c = 0;
  while (c < 5 && i >= off[c + 1]) ++c;
  if (c < 5) {
    int cnt_c = 0, ex_c = 0;
#pragma unroll
    for (int cc = 0; cc < 5; ++cc)
      if (cc == c) {
        cnt_c = cnt[cc];
        ex_c = ex[cc];
      }
    const int r = i - off[c];
    if (r >= ex_c && r < ex_c + cnt_c) {  // exactly one thread holds workgroup i
      int acc = ex_c, sacc = ex[5];
      for (int q = q0; q < q1; ++q) {
        const int k = max(s_keys[q], 0), len = s_len[q];
        const int n = npieces(k, len);
        const int wdt = p.Hkv * n;
        if (pair_cls(q, len) == c) {
          if (r < acc + wdt) {
            const int rr = r - acc;
            Piece x;
            x.b = q / nt;
            x.tile = nt - 1 - (q - x.b * nt);
            x.g = rr / n;
            x.sp = rr - x.g * n;
            x.np = n;
            x.k0 = x.sp * len;
            x.k1 = min(k, x.k0 + len);
            x.slot = sacc + x.g * n;
            x.found = 1;
            *s_pc = x;
            break;
          }
          acc += wdt;
        }
        sacc += n > 1 ? wdt : 0;
      }
    }
  }
  __syncthreads();
  pc = *s_pc;
  __syncthreads();  // the tables live in the staging buffers
}

// Staging modes (each also has an instrumented build that records the
// page and slot of every key from the address its load uses).
// kStageDma: each wave's 8-key run of a tile lies in one page (page_size a
// multiple of 8); the K/V rows are written straight into LDS by the loads
// (no staging registers, no LDS stores), with one resource for the whole K
// (V) pool and the run's position in the SGPR offset (pools under 2 GiB, so
// that offsets stay below 2^31 and an offset of 2^31 is always out of
// range).
// kStageDmaRun: the same with one buffer resource per run (pools of 2 GiB
// and more).
// kStageDmaLanes: the LDS loads of kStageDma for page sizes that are not a
// multiple of 8 (pools under 2 GiB): a wave's 8-key run may straddle pages,
// so each lane resolves its own row's page from the run's block-table
// entries and puts the whole pool offset in its own vector offset.
// kStageLanes: register staging, every lane resolving its own key (page
// sizes that are not a multiple of 8 on pools of 2 GiB and more).
enum StageMode { kStageLanes = 0, kStageDma = 3, kStageDmaRun = 4, kStageDmaLanes = 5 };

// LDS tile layout of kStageDma (64 rows x 16 chunks of 16 bytes, D = 128).
// Rows come in blocks of 4 (b = (r / 4) % 4 within a 16-row group); a block
// fills 1 KiB = 4 windows of 256 bytes (64 banks each), window w holding
// chunks 4w .. 4w + 3 of the block's 4 rows: row r % 4 in the window's 64
// bytes at 16 * (r % 4), chunk c in slot (c % 4) ^ b of them.  In shorts:
//   (r / 16) * 2048 + b * 512 + (16 * (c / 4) + 4 * (r % 4) + ((c % 4) ^ b)) * 8.
// - A K operand read (16 consecutive rows, one chunk) and a transposed V read
//   (4 rows of a block, 4 consecutive chunks) each cover all 64 banks once.
// - Every operand address is a per-lane base plus a constant: no per-read
//   address arithmetic.
// - One load instruction fills one block (4 whole rows, a contiguous 1 KiB of
//   the page), each group of 4 lanes one aligned 64-byte piece of a row, the
//   unit in which the vector memory path coalesces (see dma_tile).
__device__ __forceinline__ int dma_pos(int r, int c) {
  const int b = (r >> 2) & 3;
  return (r >> 4) * 2048 + b * 512 + (16 * (c >> 2) + 4 * (r & 3) + ((c & 3) ^ b)) * 8;
}

// LDS tile layout of the fp8 LDS-load staging (32 rows x 8 chunks of 16
// codes, D = 128): row r at byte 128 r, chunk c in slot c ^ ((r / 2) % 8).
// A K operand read (32 rows, one chunk, 8 bytes per lane) then touches every
// bank pair twice, the least that 512 bytes can.
__device__ __forceinline__ int fp8_pos(int r, int c) { return r * 128 + 16 * (c ^ ((r >> 1) & 7)); }

// The fp8 staging feeds the score product with key rows in the order pi(m)
// = 16 (m / 16) + 8 ((m / 4) % 2) + 4 ((m / 8) % 2) + m % 4 (bits 2 and 3
// of m swapped): then the 8 keys of a lane's k slot in the PV product are
// consecutive, which is what an 8-bit transposed read delivers.
__device__ __forceinline__ int fp8_key_perm(int m) {
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

typedef __attribute__((address_space(3))) void lds_void_t;
typedef int32_t i32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2_t lds_i32x2_t;

template <int D, bool DEBUG, int MODE, int RB, bool FP8>
__global__ __launch_bounds__(256, (MODE == kStageDma || MODE == kStageDmaRun ||
                                   MODE == kStageDmaLanes || FP8)
                                      ? 3
                                  : RB == 1                                ? 2
                                                                           : 1) void
prefill_kernel(LaunchParams p, int num_tiles) {
  if (contract_broken(p)) return;
  constexpr bool DMA = MODE == kStageDma || MODE == kStageDmaRun || MODE == kStageDmaLanes;
  // fp8 (E4M3) pages, D = 128: with LDS loads the codes land in LDS as they
  // are and each operand read widens them to bf16; register staging widens
  // them on their way into LDS
  static_assert(!FP8 || D == 128, "fp8 pages: D = 128");
  constexpr int EB = FP8 ? 1 : 2;  // bytes of a page element
  // keys per tile: DMA staging walks tiles of 32 keys (two 16 KiB buffers,
  // three workgroups per compute unit); the split plan's 64-key grid is a
  // multiple of it
  constexpr int BN = (DMA || FP8) ? 32 : kBN;
  constexpr int NBLK = BN / 32;    // 32-key blocks per tile
  constexpr int kRW = 32 * RB;     // packed rows per wave
  constexpr int kBM = 4 * kRW;     // packed rows per workgroup
  using TL = Tile<D>;
  static_assert(!DMA || ((D == 128 || D == 64) && RB == 1),
                "LDS-load staging: D = 128 or 64, one row block per wave");
  // rows of 128 bytes (fp8 codes with D = 128, bf16 with D = 64): the tile
  // layout of fp8_pos; rows of 256 bytes (bf16, D = 128): dma_pos
  constexpr bool ROW128 = D * EB == 128;
  // Tile buffers: padded [key][dim] rows (register staging), or four
  // separate unpadded, swizzled arrays (DMA staging: separate arrays let the
  // compiler see that a load into one buffer never feeds reads of the other).
  constexpr int kKS = DMA ? D : TL::kKStride;   // shorts per K row
  constexpr int kVS = DMA ? D : TL::kVStride;   // shorts per V row
  constexpr int kPadBuf = DMA ? 1 : 2;
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[kPadBuf][DMA ? 8 : BN * kKS];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[kPadBuf][DMA ? 8 : BN * kVS];
  // (4096 shorts at least: the planner's tables live there)
  constexpr int kDmaBuf = DMA ? (BN * D > 4096 ? BN * D : 4096) : 8;
  __shared__ __attribute__((aligned(16))) uint16_t kd0[kDmaBuf], kd1[kDmaBuf];
  __shared__ __attribute__((aligned(16))) uint16_t vd0[kDmaBuf], vd1[kDmaBuf];
  __shared__ int s_plan_red[DMA ? 32 : 1];
  __shared__ uint32_t s_arrived;
  __shared__ Piece s_pc;
  uint16_t *const kbuf0 = DMA ? kd0 : k_lds[0], *const kbuf1 = DMA ? kd1 : k_lds[kPadBuf - 1];
  uint16_t *const vbuf0 = DMA ? vd0 : v_lds[0], *const vbuf1 = DMA ? vd1 : v_lds[kPadBuf - 1];
  // the planner's tables (kSplitMaxPairs ints each) live in the staging
  // buffers: one per buffer with DMA staging, two per buffer otherwise
  int *const plan_a = reinterpret_cast<int *>(DMA ? kd0 : &k_lds[0][0]);
  int *const plan_b = reinterpret_cast<int *>(DMA ? kd1 : &k_lds[0][0] + kSplitMaxPairs * 2);
  int *const plan_c = reinterpret_cast<int *>(DMA ? vd0 : &v_lds[0][0]);
  int *const plan_d = reinterpret_cast<int *>(DMA ? vd1 : &v_lds[0][0] + kSplitMaxPairs * 2);
  int *const plan_s = DMA ? s_plan_red : plan_d + kSplitMaxPairs;
  static_assert(DMA ? sizeof(kd0) >= kSplitMaxPairs * 4 && sizeof(vd1) >= kSplitMaxPairs * 4
                    : sizeof(k_lds) >= 2 * kSplitMaxPairs * 4 &&
                          sizeof(v_lds) >= 2 * kSplitMaxPairs * 4 + 32 * 4,
                "plan tables");

  // ---- which keys of which tile: a piece of the key split (workspace
  // given), else the whole tile (heavy, late tiles first)
  int tile, g, b, k0 = 0, k1 = 0x7fffffff, np = 1, sp = 0, slot = 0;
  // the prefix launch plans pieces without a merge workspace (each piece
  // leaves its own row states)
  if (p.ws_o != nullptr || (p.prefix_pass && p.num_splits > 1)) {
    Piece pc;
    find_piece(p, num_tiles, plan_a, plan_b, plan_c, plan_d, plan_s, &s_pc, pc);
    if (!pc.found) return;  // block-uniform
    tile = pc.tile;
    g = pc.g;
    b = pc.b;
    k0 = pc.k0;
    k1 = pc.k1;
    np = pc.np;
    sp = pc.sp;
    slot = pc.slot;
  } else {  // x = tile from the last * H_kv + kv head, y = request: longest tiles first
    const int x = blockIdx.x;
    tile = num_tiles - 1 - x / p.Hkv;
    g = x - (num_tiles - 1 - tile) * p.Hkv;
    b = blockIdx.y;
  }
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  const int half = lane >> 5;       // which 8-wide k chunk / key half this lane holds
  const int ln = lane & 31;         // query row of this lane within the wave

  const int G = p.Hq / p.Hkv;
  const int ctx = launch_ctx(p, b);
  const int Lb = launch_rows(p, b);
  if (!routed_here(p, Lb)) return;  // block-uniform: a request of the other route
  const int rows_valid = G * Lb;
  // rows written: padded rows up to G * L (past query_lens as zeros); packed
  // rows of the request only; states of existing member rows (prefix launch)
  const int rows_all = (p.qsl || p.prefix_pass) ? rows_valid : G * p.L;
  const int rho0 = tile * kBM;

  // ---- this lane's query rows (one per row block)
  int rho[RB], qi[RB], qh[RB], lim[RB];
  bool row_valid[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    rho[rb] = rho0 + wave * kRW + rb * 32 + ln;
    qi[rb] = rho[rb] / G;
    qh[rb] = g * G + (rho[rb] - qi[rb] * G);
    row_valid[rb] = rho[rb] < rows_valid;
    if (p.prefix_pass && row_valid[rb]) {
      bool exists;
      launch_row(p, b, qh[rb], qi[rb], exists);
      row_valid[rb] = exists;
    }
    lim[rb] = row_valid[rb] ? (p.causal ? ctx - Lb + qi[rb] + 1 : ctx) : 0;
  }

  // ---- key ranges within [k0, k1): the workgroup's (for staging) and this
  // wave's (compute)
  const int rho_last_wg = min(rho0 + kBM, rows_valid) - 1;
  const int kend_wg = min(k1, rho_last_wg < rho0 ? 0
                              : (p.causal ? ctx - Lb + rho_last_wg / G + 1 : ctx));
  const int rho_first_w = rho0 + wave * kRW;
  const int rho_last_w = min(rho_first_w + kRW, rows_valid) - 1;
  const int kend_w = min(k1, rho_last_w < rho_first_w ? 0
                             : (p.causal ? ctx - Lb + rho_last_w / G + 1 : ctx));
  const int kfull_w = rho_last_w < rho_first_w ? 0
                      : (p.causal ? ctx - Lb + rho_first_w / G + 1 : ctx);  // keys below: unmasked
  const int kt0 = k0 / BN;  // first tile (k0 is a multiple of 64)
  const int ntiles = kend_wg > k0 ? (kend_wg - k0 + BN - 1) / BN : 0;
  const bool counts = DEBUG && rows_valid > 0 && (rows_valid - 1) / kBM == tile;

  // ---- Q as the B operand of S^T = K Q^T: dims kk*16 + half*8 .. +8
  uint4 q[RB][TL::kKSteps];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    bool exists;
    const size_t qr = row_valid[rb] ? launch_row(p, b, qh[rb], qi[rb], exists) : 0;
    const uint16_t *qp = reinterpret_cast<const uint16_t *>(p.q) + qr * D + half * 8;
#pragma unroll
    for (int kk = 0; kk < TL::kKSteps; ++kk)
      q[rb][kk] = row_valid[rb] ? *reinterpret_cast<const uint4 *>(qp + kk * 16)
                                : make_uint4(0, 0, 0, 0);
  }

  // ---- staging of one K/V tile: thread -> (key kr*KPR + tid / CH, chunk tid % CH)
  const uint16_t *kp = reinterpret_cast<const uint16_t *>(p.kp);
  const uint16_t *vp = reinterpret_cast<const uint16_t *>(p.vp);
  const uint8_t *kp8 = reinterpret_cast<const uint8_t *>(p.kp);  // fp8 pages
  const uint8_t *vp8 = reinterpret_cast<const uint8_t *>(p.vp);
  // the prefix launch reads the table of the group's first member
  const int32_t *bt = p.bt + (size_t)(p.prefix_pass ? p.grp_start[b] : b) * p.max_pages;
  const int chunk = tid % TL::kChunks;
  const int key_in_round = tid / TL::kChunks;
  // one staged K/V tile in registers: 8 bf16 elements per lane and round,
  // or for fp8 pages their 8 codes, widened only when stored to LDS (a
  // conversion next to the load would wait for it at once)
  using StageWord = typename std::conditional<FP8, uint2, uint4>::type;
  constexpr int kRounds = BN / TL::kKeysPerRound;  // staging rounds per tile
  struct Stage {
    StageWord k[DMA ? 1 : kRounds], v[DMA ? 1 : kRounds];
  };

  // The block table is read-only for the whole call: reading it through the
  // constant address space lets wave-uniform entries come in by scalar loads.
  typedef const __attribute__((address_space(4))) int32_t *const_i32_ptr;
  const const_i32_ptr btc = (const_i32_ptr)bt;
  const long long page_bytes = (long long)p.Hkv * p.ps * D * EB;
  const long long head_bytes = (long long)g * p.ps * D * EB;
  const char *kp_bytes = reinterpret_cast<const char *>(p.kp);
  const char *vp_bytes = reinterpret_cast<const char *>(p.vp);
  int pass = 0;  // 1: the walk again with exact row maxima
  // Debug record of logical key j, decoded from the byte offset into the
  // pool that this thread's load of the key's first 16-byte chunk actually
  // uses: page, kv head and slot follow from the layout [num_pages, H_kv,
  // page_size, D] alone, so the trace observes the staging's own address
  // arithmetic.  The visit is counted under the kv head the offset points at.
  auto record = [&](int j, long long byte) {
    if constexpr (DEBUG) {
      const long long head_row = (long long)p.ps * D * EB;  // bytes of one page of one head
      if (counts && pass == 0 && j < kend_wg && byte % (D * EB) == 0) {
        const long long ph = byte / head_row;               // page * H_kv + head
        const int slot = (int)((byte - ph * head_row) / (D * EB));
        const int page = (int)(ph / p.Hkv);
        const int head = (int)(ph - (long long)page * p.Hkv);
        const size_t cap = (size_t)p.max_pages * p.ps;
        if (g == 0) {
          p.dbg_trace[((size_t)b * cap + j) * 2 + 0] = page;
          p.dbg_trace[((size_t)b * cap + j) * 2 + 1] = slot;
        }
        atomicAdd(&p.dbg_visits[((size_t)b * p.Hkv + head) * cap + j], 1);
      }
    }
  };
  const int pool_bytes = (int)((long long)p.num_pages * page_bytes);  // pools under 2 GiB
  const __amdgpu_buffer_rsrc_t pool_k = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char *>(kp_bytes), (short)0, pool_bytes, kBufferRsrcWord3);
  const __amdgpu_buffer_rsrc_t pool_v = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char *>(vp_bytes), (short)0, pool_bytes, kBufferRsrcWord3);
  // DMA staging: wave w loads keys R*w .. R*w + R - 1 of a tile (R = BN / 4,
  // within one page), i.e. blocks Bw .. Bw + R/4 - 1 of 4 rows (Bw = R/4 * w);
  // instruction j fills block B = Bw + j: lane l writes slot l of that 1 KiB
  // with chunk 4 * (l / 16) + ((l % 4) ^ (B % 4)) of row 4B + (l / 4) % 4
  // (see dma_pos).  The per-lane offsets are fixed for the whole walk; the
  // run's page and slot are advanced by BN keys per tile.
  constexpr int kDmaRows = BN / 4;          // keys per wave and tile
  // load instructions per wave, K and V each: 4 rows of bf16 or 8 rows of
  // fp8 codes per 1 KiB
  constexpr int kDmaRowsPerLoad = ROW128 ? 8 : 4;
  constexpr int kDmaBlocks = kDmaRows / kDmaRowsPerLoad;
  const int dma_row = ROW128 ? lane >> 3 : (lane >> 2) & 3;
  int dma_voff[kDmaBlocks];
#pragma unroll
  for (int j = 0; j < kDmaBlocks; ++j) {
    if constexpr (ROW128) {
      // lane l fills slot l % 8 of row l / 8 of the wave's 8 rows (fp8_pos)
      const int r = kDmaRows * wave + dma_row;
      dma_voff[j] = dma_row * (D * EB) + 16 * ((lane & 7) ^ ((r >> 1) & 7));
    } else {
      const int blk4 = (kDmaBlocks * wave + j) & 3;
      dma_voff[j] = (4 * j + dma_row) * (D * 2) + (4 * (lane >> 4) + ((lane & 3) ^ blk4)) * 16;
    }
  }
  int dma_lp = 0, dma_slot = 0;
  auto dma_tile = [&](int T, uint16_t *kdst, uint16_t *vdst) {
    const int run0 = T * BN + kDmaRows * wave;  // first key of this wave's run
    const bool live = run0 < kend_wg;           // wave-uniform
    if constexpr (MODE == kStageDmaLanes) {
      // the run's keys lie on at most kDmaRows pages from its first one on;
      // lane row r (run0 + r) is q = (s0 + r) / ps pages further
      const int lp0 = run0 / p.ps;
      const int s0 = run0 - lp0 * p.ps;
      int ent[kDmaRows];
#pragma unroll
      for (int i = 0; i < kDmaRows; ++i) ent[i] = live ? btc[min(lp0 + i, p.max_pages - 1)] : 0;
#pragma unroll
      for (int j = 0; j < kDmaBlocks; ++j) {
        const int r = kDmaRowsPerLoad * j + dma_row;
        int q = 0;
#pragma unroll
        for (int m = 1; m < kDmaRows; ++m) q += s0 + r >= m * p.ps ? 1 : 0;
        int pg = ent[0];
#pragma unroll
        for (int m = 1; m < kDmaRows; ++m) pg = q == m ? ent[m] : pg;
        const int slot = s0 + r - q * p.ps;
        const int coff = dma_voff[j] - r * (D * EB);  // the lane's chunk within the row
        const int voff = run0 + r < kend_wg
                             ? pg * (int)page_bytes + (int)head_bytes + slot * (D * EB) + coff
                             : (int)0x80000000u;
        const int dst = (kDmaBlocks * wave + j) * 512;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(pool_k, (lds_void_t *)(kdst + dst), 16, voff, 0,
                                                 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(pool_v, (lds_void_t *)(vdst + dst), 16, voff, 0,
                                                 0, 0);
        if constexpr (DEBUG)
          if (voff >= 0) record(run0 + r, voff);
      }
      return;
    }
    const int page = live ? btc[min(dma_lp, p.max_pages - 1)] : 0;
    // pool-wide resources with the run in the scalar offset, or (pools of
    // 2 GiB and more) resources of the run itself, empty past the last key
    __amdgpu_buffer_rsrc_t rk = pool_k, rv = pool_v;
    int soff = 0;
    if constexpr (MODE == kStageDmaRun) {
      const long long off =
          (long long)page * page_bytes + head_bytes + (long long)dma_slot * (D * EB);
      const int nrec = live ? kDmaRows * D * EB : 0;
      rk = __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(kp_bytes + off), (short)0, nrec,
                                             kBufferRsrcWord3);
      rv = __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(vp_bytes + off), (short)0, nrec,
                                             kBufferRsrcWord3);
    } else {
      soff = page * (int)page_bytes + (int)head_bytes + dma_slot * (D * EB);
    }
    auto load = [&](int j, int voff) {
      const int dst = (kDmaBlocks * wave + j) * 512;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void_t *)(kdst + dst), 16, voff, soff, 0,
                                               0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void_t *)(vdst + dst), 16, voff, soff, 0,
                                               0);
      if constexpr (DEBUG) {
        // byte offset of this lane's chunk from the pool base: the resource
        // base (per-run resources) or the scalar offset (pool-wide), plus
        // the lane offset
        long long base = soff;
        if constexpr (MODE == kStageDmaRun)
          base = (long long)page * page_bytes + head_bytes + (long long)dma_slot * (D * EB);
        if (live && voff >= 0) record(run0 + kDmaRowsPerLoad * j + dma_row, base + voff);
      }
    };
    if (run0 + kDmaRows <= kend_wg) {  // wave-uniform: the whole run is live
#pragma unroll
      for (int j = 0; j < kDmaBlocks; ++j) load(j, dma_voff[j]);
    } else {
      // rows past the workgroup's last key read as zeros (stale slots may
      // hold anything, NaN included)
#pragma unroll
      for (int j = 0; j < kDmaBlocks; ++j)
        load(j, run0 + kDmaRowsPerLoad * j + dma_row < kend_wg ? dma_voff[j] : (int)0x80000000u);
    }
    dma_slot += BN;
    while (dma_slot >= p.ps) {
      dma_slot -= p.ps;
      ++dma_lp;
    }
  };
  auto stage_load = [&](int kt, Stage &st) {
#pragma unroll
    for (int r = 0; r < kRounds; ++r) {
      const int j = kt * BN + r * TL::kKeysPerRound + key_in_round;
      if (j < kend_wg) {
        const int lp = j / p.ps;
        const int page = bt[lp];
        const int slot = j - lp * p.ps;
        const size_t off = (((size_t)page * p.Hkv + g) * p.ps + slot) * D + chunk * 8;
        if constexpr (FP8) {
          st.k[r] = *reinterpret_cast<const uint2 *>(kp8 + off);
          st.v[r] = *reinterpret_cast<const uint2 *>(vp8 + off);
        } else {
          st.k[r] = *reinterpret_cast<const uint4 *>(kp + off);
          st.v[r] = *reinterpret_cast<const uint4 *>(vp + off);
        }
        record(j, (long long)off * EB);
      } else {
        st.k[r] = StageWord{};  // never loaded: zeros keep masked math finite
        st.v[r] = StageWord{};
      }
    }
  };
  auto stage_store = [&](uint16_t *kdst, uint16_t *vdst, const Stage &st) {
    if constexpr (!DMA) {
#pragma unroll
      for (int r = 0; r < kRounds; ++r) {
        const int key = r * TL::kKeysPerRound + key_in_round;
        if constexpr (FP8) {
          *reinterpret_cast<uint4 *>(&kdst[key * kKS + chunk * 8]) =
              fp8x8_to_bf16x8(st.k[r].x, st.k[r].y);
          *reinterpret_cast<uint4 *>(&vdst[key * kVS + chunk * 8]) =
              fp8x8_to_bf16x8(st.v[r].x, st.v[r].y);
        } else {
          *reinterpret_cast<uint4 *>(&kdst[key * kKS + chunk * 8]) = st.k[r];
          *reinterpret_cast<uint4 *>(&vdst[key * kVS + chunk * 8]) = st.v[r];
        }
      }
    }
  };

  // ---- state of this lane's query rows
  f32x16_t o[RB][TL::kMBlocks];
  float m_ref[RB], m_seen[RB], l_run[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m_ref[rb] = kMinM;
    m_seen[rb] = kMinM;
  }
  // score multiplier in base-2 units (fp8 pages: times k_scale)
  const float c = FP8 ? p.scale_log2 * p.k_scale : p.scale_log2;

  // Register staging: with one row block per wave, two sets (set A holds
  // even tiles, set B odd ones) so that loads run two tiles ahead; with two
  // row blocks a tile is long enough for loads one tile ahead, in one set.
  // fp8 codes take one set too: at three workgroups per CU a second set
  // spills, and loads one 32-key tile ahead measured faster than that.
  constexpr bool kTwoSets = RB == 1 && !FP8;
  Stage sa, sb;
 for (; pass < 2; ++pass) {
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
    for (int mb = 0; mb < TL::kMBlocks; ++mb)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[rb][mb][i] = 0.f;
    l_run[rb] = 0.f;
  }
  if constexpr (DMA) {
    // tile kt0 goes to buffer 0; the first step waits for it (no load is
    // issued that the walk does not wait for: LDS must not be written after
    // the workgroup ends)
    dma_lp = (k0 + kDmaRows * wave) / p.ps;
    dma_slot = (k0 + kDmaRows * wave) - dma_lp * p.ps;
    if (ntiles > 0) dma_tile(kt0, kbuf0, vbuf0);
  } else {
    if (ntiles > 0) {
      stage_load(kt0, sa);
      stage_store(kbuf0, vbuf0, sa);
    }
    if (kTwoSets && ntiles > 1) stage_load(kt0 + 1, sb);
    // the query and tile-0 loads are complete here; tile 1 stays in flight
    __builtin_amdgcn_s_waitcnt(kWaitVmcntOlderThan8);
    __syncthreads();
  }

  // One tile: prefetch tile kt + 2 into `ld` (its set is free: tile kt was
  // stored to LDS one tile ago), compute tile kt, then store tile kt + 1
  // (loaded into `st` one tile ago) to the other LDS buffer.
  // kStageDma operand bases (block 0, first steps): K for even / odd k-steps
  // (2 kk + half), V rows kb .. kb + 3 and kb + 8 .. kb + 11 of the
  // transposed reads; every other read adds a constant (see dma_pos)
  int k_dma[2] = {0, 0}, v_dma[2] = {0, 0};
  // fp8 LDS loads: K row pi(lane % 32) and its chunk slot key; V rows for
  // the 8-bit transposed reads (lane 2j + c of a 16-lane group points at
  // 8 codes of row j of its 8 keys, columns + 8 c) and their slot key
  int k8_row = 0, k8_key = 0, v8_off = 0, v8_key = 0;
  // bf16 rows of 128 bytes (D = 64): K row lane % 32, chunk 2 kk + half; V
  // rows of the two 16-bit transposed reads and their chunk slot keys
  int k64_row = 0, k64_key = 0, v64_off = 0, v64_c = 0, v64_key1 = 0, v64_key2 = 0;
  if constexpr (DMA && ROW128 && !FP8) {
    k64_row = ln * 128;
    k64_key = (ln >> 1) & 7;
    const int src = lane & 15;
    const int r1 = half * 4 + (src >> 2);  // the second read: row r1 + 8
    v64_off = r1 * 128 + 8 * (src & 1);
    v64_c = 2 * ((lane >> 4) & 1) + ((src & 3) >> 1);
    v64_key1 = (r1 >> 1) & 7;
    v64_key2 = ((r1 + 8) >> 1) & 7;
  }
  if constexpr (DMA && FP8) {
    const int kr = fp8_key_perm(ln);
    k8_row = kr * 128 + 8 * half;
    k8_key = (kr >> 1) & 7;
    const int rv = ((lane & 15) >> 1) + 8 * (lane >> 5);  // key within the 16-key step
    v8_off = rv * 128 + 8 * (lane & 1);
    v8_key = (rv >> 1) & 7;                            // rows 16 hf + rv share it
  } else if constexpr (DMA) {
    k_dma[0] = dma_pos(ln, half);
    k_dma[1] = dma_pos(ln, 2 + half);
    const int src = lane & 15;
    const int d0 = ((lane >> 4) & 1) * 16 + 4 * (src & 3);
    v_dma[0] = dma_pos(half * 4 + (src >> 2), d0 >> 3) + (d0 & 7);
    v_dma[1] = dma_pos(half * 4 + (src >> 2) + 8, d0 >> 3) + (d0 & 7);
  }
  const int kt_end = kt0 + ntiles;
  // kc/vc: the buffers of tile kt; kn/vn: the other pair (tile kt + 1)
  auto tile_step = [&](int kt, Stage &ld, const Stage &st, const uint16_t *kc, const uint16_t *vc,
                       uint16_t *kn, uint16_t *vn) {
    const bool more = kt + 1 < kt_end;
    if constexpr (DMA) {
      // tile kt is in LDS once every wave's loads of it are done; after the
      // barrier no wave still reads tile kt - 1, whose buffers take tile
      // kt + 1 (the loads write LDS through the memory path, not in order
      // with LDS reads, so every wave's reads are complete before it
      // arrives: lgkmcnt(0))
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
      __syncthreads();
    } else if constexpr (kTwoSets) {
      if (kt + 2 < kt_end) stage_load(kt + 2, ld);
    } else {
      if (more) stage_load(kt + 1, ld);
    }

    if (kt * BN < kend_w) {
      // The tile's 32-key blocks are processed one after the other (scores,
      // softmax, PV), which keeps the score and P registers of a single
      // block live.
#pragma unroll
      for (int blk = 0; blk < NBLK; ++blk) {
        // -- S^T of this block; each K operand read from LDS feeds the RB
        //    row blocks
        f32x16_t s[RB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int i = 0; i < 16; ++i) s[rb][i] = 0.f;
        const uint16_t *krow = kc + (blk * 32 + ln) * kKS;
#pragma unroll
        for (int kk = 0; kk < TL::kKSteps; ++kk) {
          uint4 a;
          if constexpr (DMA && FP8) {
            const uint8_t *kb8 = reinterpret_cast<const uint8_t *>(kc);
            const uint2 w = *reinterpret_cast<const uint2 *>(kb8 + k8_row + 16 * (kk ^ k8_key));
            a = fp8x8_to_bf16x8(w.x, w.y);
          } else if constexpr (DMA && ROW128) {
            const uint8_t *kb8 = reinterpret_cast<const uint8_t *>(kc);
            a = *reinterpret_cast<const uint4 *>(kb8 + k64_row +
                                                 16 * ((2 * kk + half) ^ k64_key));
          } else {
            const uint16_t *ka = DMA ? kc + k_dma[kk & 1] + blk * 4096 + (kk >> 1) * 128
                                     : krow + kk * 16 + half * 8;
            a = *reinterpret_cast<const uint4 *>(ka);
          }
#pragma unroll
          for (int rb = 0; rb < RB; ++rb)
            s[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(q[rb][kk]),
                                                            s[rb], 0, 0, 0);
        }
        // DMA staging: the next tile's loads go out once this block's K
        // operands have been read (they write the other buffer)
        if (DMA && blk == 0 && more) dma_tile(kt + 1, kn, vn);
        // -- mask keys at or past each row's limit (diagonal / tail blocks only)
        if (kt * BN + (blk + 1) * 32 > kfull_w) {
#pragma unroll
          for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int key =
                  DMA && FP8 ? kt * BN + blk * 32 + fp8_key_perm((i >> 2) * 8 + half * 4 + (i & 3))
                             : kt * BN + blk * 32 + (i >> 2) * 8 + half * 4 + (i & 3);
              if (key >= lim[rb]) s[rb][i] = kNegInf;
            }
        }
        // -- online softmax update of each row
        uint32_t pb[RB][8];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          float mx = max3(s[rb][0], s[rb][1], s[rb][2]);
#pragma unroll
          for (int i = 3; i < 15; i += 2) mx = max3(mx, s[rb][i], s[rb][i + 1]);
          mx = pair_max(max3(mx, s[rb][15], s[rb][15])) * c;
          if (pass == 0 && kt == kt0 && blk == 0) m_ref[rb] = fmaxf(mx, kMinM);
          m_seen[rb] = fmaxf(m_seen[rb], mx);
          // the row sum adds the bf16 weights that PV multiplies (dot2 with
          // (1, 1): exact products, fp32 sums), in two chains
          float psum0 = 0.f, psum1 = 0.f;
#pragma unroll
          for (int i = 0; i < 16; i += 2) {
            const float p0 = fast_exp2(fmaf(s[rb][i], c, -m_ref[rb]));  // masked -> 0
            const float p1 = fast_exp2(fmaf(s[rb][i + 1], c, -m_ref[rb]));
            pb[rb][i >> 1] = cvt_pk_bf16(p0, p1);
            if (i & 2)
              psum1 = dot2_bf16(pb[rb][i >> 1], kBf16OnePair, psum1);
            else
              psum0 = dot2_bf16(pb[rb][i >> 1], kBf16OnePair, psum0);
          }
          l_run[rb] += psum0 + psum1;
        }

        // -- O^T += V^T P^T over the block's two 16-key steps; each V^T
        //    operand feeds the RB row blocks
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          uint4 bop[RB];
#pragma unroll
          for (int rb = 0; rb < RB; ++rb)
            bop[rb] = make_uint4(pb[rb][hf * 4 + 0], pb[rb][hf * 4 + 1], pb[rb][hf * 4 + 2],
                                 pb[rb][hf * 4 + 3]);
          // keys of the two 4-key runs this lane's k slots stand for
          const int kb = blk * 32 + hf * 16 + half * 4;
          const int src = lane & 15;  // transpose read: source lane j reads row kb + j/4, cols +4*(j%4)
#pragma unroll
          for (int mb = 0; mb < TL::kMBlocks; ++mb) {
            const int d0 = mb * 32 + ((lane >> 4) & 1) * 16 + 4 * (src & 3);
            const int vr = kb + (src >> 2);
            uint4 aop;
            if constexpr (DMA && FP8) {
              // 8 codes of the lane's column for keys 16 hf + 8 half .. + 7
              // (chunk 2 mb + (lane / 16) % 2 of their rows), widened to bf16
              const uint8_t *vb8 = reinterpret_cast<const uint8_t *>(vc);
              const int c8 = 2 * mb + ((lane >> 4) & 1);
              const i32x2_t t = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                  (lds_i32x2_t *)(vb8 + hf * 16 * 128 + v8_off + 16 * (c8 ^ v8_key)));
              aop = fp8x8_to_bf16x8((uint32_t)t[0], (uint32_t)t[1]);
            } else if constexpr (DMA && ROW128) {
              // keys 16 hf + 4 half + 0..3 and + 8, columns mb * 32 + 16 (lane /
              // 16 % 2) + 4 (lane % 4) of the lane's transposed reads
              const uint8_t *vb8 = reinterpret_cast<const uint8_t *>(vc);
              const int c = 4 * mb + v64_c;
              const s16x4_t t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                  (lds_s16x4_t *)(vb8 + hf * 2048 + v64_off + 16 * (c ^ v64_key1)));
              const s16x4_t t2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                  (lds_s16x4_t *)(vb8 + hf * 2048 + v64_off + 1024 + 16 * (c ^ v64_key2)));
              aop = make_uint4((uint32_t)(uint16_t)t1[0] | ((uint32_t)(uint16_t)t1[1] << 16),
                               (uint32_t)(uint16_t)t1[2] | ((uint32_t)(uint16_t)t1[3] << 16),
                               (uint32_t)(uint16_t)t2[0] | ((uint32_t)(uint16_t)t2[1] << 16),
                               (uint32_t)(uint16_t)t2[2] | ((uint32_t)(uint16_t)t2[3] << 16));
            } else {
              const int vo = blk * 4096 + hf * 2048 + mb * 128;  // kStageDma
              const uint16_t *r1 = DMA ? vc + v_dma[0] + vo : vc + vr * kVS + d0;
              const uint16_t *r2 = DMA ? vc + v_dma[1] + vo : vc + (vr + 8) * kVS + d0;
              const s16x4_t t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t *)r1);
              const s16x4_t t2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t *)r2);
              aop = make_uint4((uint32_t)(uint16_t)t1[0] | ((uint32_t)(uint16_t)t1[1] << 16),
                               (uint32_t)(uint16_t)t1[2] | ((uint32_t)(uint16_t)t1[3] << 16),
                               (uint32_t)(uint16_t)t2[0] | ((uint32_t)(uint16_t)t2[1] << 16),
                               (uint32_t)(uint16_t)t2[2] | ((uint32_t)(uint16_t)t2[3] << 16));
            }
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
              o[rb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                  as_bf16x8(aop), as_bf16x8(bop[rb]), o[rb][mb], 0, 0, 0);
          }
        }
      }
    }

    if constexpr (DMA) {
      if (kt * BN >= kend_w && more) dma_tile(kt + 1, kn, vn);  // no compute in this tile
    } else {
      if (more) stage_store(kn, vn, st);
      __syncthreads();
    }
  };
  // unrolled by two: each half has its own staging set and LDS buffers
  Stage &s2 = kTwoSets ? sb : sa;
  for (int kt = kt0; kt < kt_end; kt += 2) {
    tile_step(kt, sa, s2, kbuf0, vbuf0, kbuf1, vbuf1);
    if (kt + 1 < kt_end) tile_step(kt + 1, s2, sa, kbuf1, vbuf1, kbuf0, vbuf0);
  }
  if constexpr (DMA) __syncthreads();  // the last tile is read before a rerun restages
  // weights past 2^16 anywhere in the workgroup: walk again from the exact maxima
  bool over = false;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) over |= m_seen[rb] > m_ref[rb] + kRefSlack;
  if (pass == 1 || !__syncthreads_or(over)) break;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) m_ref[rb] = m_seen[rb];
 }

  // ---- a piece of a split tile: publish this piece's state; the last piece
  // to arrive merges all of them and writes the output
  if (np > 1 && !p.prefix_pass) {
    if constexpr (RB == 1) {
      constexpr int kAcc = TL::kMBlocks * 16;  // accumulators per thread (D / 2)
      auto slot_o = [&](int s) {
        return __builtin_amdgcn_make_buffer_rsrc(p.ws_o + (size_t)(slot + s) * kAcc * 256,
                                                 (short)0, kAcc * 256 * 4, kBufferRsrcWord3);
      };
      auto slot_m = [&](int s) {
        return __builtin_amdgcn_make_buffer_rsrc(p.ws_lse + (size_t)(slot + s) * 2 * 256,
                                                 (short)0, 2 * 256 * 4, kBufferRsrcWord3);
      };
      // [value / 4][thread][4]: every 16-byte store and load of a wave is
      // one coalesced 1 KiB row; written through to memory for the merging
      // workgroup, which may run on another XCD.  A wave whose rows all lie
      // past the request's rows publishes and merges nothing (those rows
      // are written as zeros, or not at all).
      const bool live_w = rho_first_w < rows_valid;  // wave-uniform
      auto off4 = [&](int mb, int j) { return ((mb * 4 + j) * 256 + tid) * 16; };
      if (live_w) {
        const auto ro = slot_o(sp);
        const auto rm = slot_m(sp);
#pragma unroll
        for (int mb = 0; mb < TL::kMBlocks; ++mb)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const f32x16_t &om = o[0][mb];
            const u32x4_t v = {__float_as_uint(om[4 * j]), __float_as_uint(om[4 * j + 1]),
                               __float_as_uint(om[4 * j + 2]), __float_as_uint(om[4 * j + 3])};
            __builtin_amdgcn_raw_buffer_store_b128(v, ro, off4(mb, j), 0, kSysScope);
          }
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(m_ref[0]), rm, tid * 4, 0, kSysScope);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(l_run[0]), rm, (256 + tid) * 4, 0,
                                              kSysScope);
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the state is in memory
      __syncthreads();
      if (tid == 0)
        s_arrived = __hip_atomic_fetch_add(p.counters + slot, 1u, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
      __syncthreads();
      if (s_arrived != (uint32_t)(np - 1)) return;  // block-uniform
      asm volatile("" ::: "memory");
      auto ld = [](__amdgpu_buffer_rsrc_t r, int off) {
        return __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kSysScope));
      };
      // Every piece, this one included, is read back and summed in piece
      // order: the result does not depend on which piece arrived last.  The
      // maxima come first, 16 pieces per batch of loads in flight together
      // (a slot past the last piece reads as empty: its offset lies outside
      // the resource); then each piece costs one round trip to memory.
      if (live_w) {
        float M = kMinM;
        for (int s0 = 0; s0 < np; s0 += 16) {
          float ms[16];
#pragma unroll
          for (int k = 0; k < 16; ++k)
            ms[k] = ld(slot_m(s0 + k), s0 + k < np ? tid * 4 : (int)0x80000000u);
#pragma unroll
          for (int k = 0; k < 16; ++k) M = fmaxf(M, s0 + k < np ? ms[k] : kMinM);
        }
        m_ref[0] = M;  // the merged state's reference
        l_run[0] = 0.f;
#pragma unroll
        for (int mb = 0; mb < TL::kMBlocks; ++mb)
#pragma unroll
          for (int i = 0; i < 16; ++i) o[0][mb][i] = 0.f;
        for (int s2 = 0; s2 < np; ++s2) {
          const auto ro = slot_o(s2);
          const auto rm = slot_m(s2);
          const float f = fast_exp2(ld(rm, tid * 4) - M);
          l_run[0] = fmaf(f, ld(rm, (256 + tid) * 4), l_run[0]);
#pragma unroll
          for (int mb = 0; mb < TL::kMBlocks; ++mb)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(ro, off4(mb, j), 0, kSysScope);
#pragma unroll
              for (int e = 0; e < 4; ++e)
                o[0][mb][4 * j + e] = fmaf(f, __uint_as_float(v[e]), o[0][mb][4 * j + e]);
            }
        }
      }
      if (tid == 0) __hip_atomic_store(p.counters + slot, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }

  // ---- prefix launch: this piece's state of each member row, by the
  // row's output index: normalised output (fp32) and natural-log
  // log-sum-exp, in piece slot sp of the row; piece 0 records the count
  if (p.prefix_pass) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const float l_tot = pair_sum(l_run[rb]);  // uniform: every lane of the wave takes part
      if (!row_valid[rb]) continue;
      bool exists;
      const size_t orow = launch_row(p, b, qh[rb], qi[rb], exists);
      const size_t ps_row = orow * kPrefixPieces + sp;
      const float inv = l_tot > 0.f ? (FP8 ? p.v_scale : 1.f) / l_tot : 0.f;
      float *po = p.pre_o + ps_row * D;
#pragma unroll
      for (int mb = 0; mb < TL::kMBlocks; ++mb)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int d = mb * 32 + i4 * 8 + half * 4;
          const f32x16_t &om = o[rb][mb];
          *reinterpret_cast<float4 *>(po + d) =
              make_float4(om[i4 * 4 + 0] * inv, om[i4 * 4 + 1] * inv, om[i4 * 4 + 2] * inv,
                          om[i4 * 4 + 3] * inv);
        }
      if (half == 0) {
        p.pre_lse[ps_row] = l_tot > 0.f ? (m_ref[rb] + __log2f(l_tot)) * kLn2 : kNegInf;
        if (sp == 0) p.pre_n[orow] = np;
      }
    }
    return;
  }

  // ---- finalize: O = O^T / l, rounded to bf16; padding rows get zeros
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const float l_tot = pair_sum(l_run[rb]);  // uniform: every lane of the wave takes part
    if (rho[rb] < rows_all) {
      // fp8 pages: the values carry v_scale, applied once here
      const float inv = (row_valid[rb] && l_tot > 0.f) ? (FP8 ? p.v_scale : 1.f) / l_tot : 0.f;
      uint16_t *op = reinterpret_cast<uint16_t *>(p.out) + query_row(p, b, qh[rb], qi[rb]) * D;
#pragma unroll
      for (int mb = 0; mb < TL::kMBlocks; ++mb)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int d = mb * 32 + i4 * 8 + half * 4;
          const f32x16_t &om = o[rb][mb];
          const uint2 w = make_uint2(cvt_pk_bf16(om[i4 * 4 + 0] * inv, om[i4 * 4 + 1] * inv),
                                     cvt_pk_bf16(om[i4 * 4 + 2] * inv, om[i4 * 4 + 3] * inv));
          *reinterpret_cast<uint2 *>(op + d) = w;
        }
    }
  }
}

template <int D, int RB>
hipError_t launch_rb(const LaunchParams &p, hipStream_t stream) {
  const int G = p.Hq / p.Hkv;
  const int bm = 128 * RB;
  const int tiles = (G * p.L + bm - 1) / bm;
  // key split: one workgroup per piece, at most one per tile plus half the
  // slots (see find_piece)
  const bool split = p.ws_o != nullptr || (p.prefix_pass && p.num_splits > 1);
  // pairs that can have rows: every (request, tile), or with packed rows of
  // known total T at most floor(G T / bm) + (requests with rows): each such
  // request adds at most one partial tile, and a request of the prefill
  // route of a ragged call has two rows or more (the planner orders the
  // pairs without rows last, so the workgroups cover the others)
  long long pairs = (long long)tiles * p.B;
  if (split && p.qsl && p.num_tokens > 0 && !p.prefix_pass) {
    const long long T = p.num_tokens;
    const long long with_rows = min((long long)p.B, p.route == 2 ? T / 2 : T);
    pairs = min(pairs, (long long)G * T / bm + with_rows);
  }
  dim3 grid = split ? dim3((unsigned)(pairs * p.Hkv + max(1, p.num_splits / 2)))
                    : dim3((unsigned)((long long)tiles * p.Hkv), p.B);
  // the debug outputs select the instrumented build of the same staging mode
  const bool debug = p.dbg_trace || p.dbg_visits;
  auto go = [&](auto dbg, auto fp8) {
    constexpr bool DBG = decltype(dbg)::value;
    constexpr bool F8 = decltype(fp8)::value;
    // LDS-load staging (one row block per wave): 8-key runs inside a page
    // with the page in a scalar offset (or, pools of 2 GiB and more, one
    // resource per run); other page sizes resolve each row's page, and on
    // pools of 2 GiB and more stage through registers
    static_assert((D == 128 || D == 64) && RB == 1, "LDS-load staging");
    const long long pool = (long long)p.num_pages * p.Hkv * p.ps * D * (F8 ? 1 : 2);
    const bool runs = p.ps % 8 == 0;
    if (pool < (1ll << 31)) {
      if (runs)
        hipLaunchKernelGGL((prefill_kernel<D, DBG, kStageDma, RB, F8>), grid, dim3(256), 0,
                           stream, p, tiles);
      else
        hipLaunchKernelGGL((prefill_kernel<D, DBG, kStageDmaLanes, RB, F8>), grid, dim3(256), 0,
                           stream, p, tiles);
    } else if (runs) {
      hipLaunchKernelGGL((prefill_kernel<D, DBG, kStageDmaRun, RB, F8>), grid, dim3(256), 0,
                         stream, p, tiles);
    } else {
      hipLaunchKernelGGL((prefill_kernel<D, DBG, kStageLanes, RB, F8>), grid, dim3(256), 0,
                         stream, p, tiles);
    }
  };
  using yes = std::integral_constant<bool, true>;
  using no = std::integral_constant<bool, false>;
  if (p.kv_fp8) {
    if constexpr (D == 128) {  // fp8 pages come with D = 128 only
      if (debug)
        go(yes(), yes());
      else
        go(no(), yes());
    } else {
      return hipErrorInvalidValue;
    }
  } else if (debug) {
    go(yes(), no());
  } else {
    go(no(), no());
  }
  return hipGetLastError();
}

// One row block per wave (the key split assumes it): two row blocks halve
// the LDS traffic per flop but
// need the accumulation registers of 64 rows, which leaves one wave per SIMD
// and measured slower than two waves of one row block each.
template <int D>
hipError_t launch_d(const LaunchParams &p, hipStream_t stream) {
  return launch_rb<D, 1>(p, stream);
}

}  // namespace

hipError_t launch_prefill_mfma(const LaunchParams &p, hipStream_t stream) {
  return p.D == 64 ? launch_d<64>(p, stream) : launch_d<128>(p, stream);
}

}  // namespace pa
