// K/V write path: every new token's key and value rows go to their physical
// slots in the page pool ("Reading vLLM's PagedAttention Kernel", section
// 3.2: the write side scatters tokens to flat slots page * page_size +
// offset, the read side gathers them back through the block table).
//
// One thread moves 16 bytes: a row of head_dim elements (128, 256 or 512
// bytes) is LANES consecutive threads, so a wave copies 1 KiB of source rows
// per instruction and each row lands as one contiguous run of its page.
// The slot of a token is read by the LANES threads of each of its rows (one
// cached load).  Tokens with a negative or out-of-pool slot are skipped.
// HBM bound: every byte is read once and written once.
#include "pa_write.h"

namespace pa {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

template <int LANES>
__global__ __launch_bounds__(256) void append_kernel(AppendParams p) {
  constexpr int kRowsPerBlock = 256 / LANES;
  const int part = threadIdx.x % LANES;  // 16-byte piece of the row
  const long long rows = (long long)p.tokens * p.Hkv;
  const long long stride = (long long)gridDim.x * kRowsPerBlock;
  for (long long r = (long long)blockIdx.x * kRowsPerBlock + threadIdx.x / LANES; r < rows;
       r += stride) {
    const int t = (int)(r / p.Hkv);
    const int h = (int)(r - (long long)t * p.Hkv);
    const int s = p.slots[t];
    if (s < 0 || s >= p.num_slots) continue;
    const int page = s / p.ps;
    const int off = s - page * p.ps;
    const size_t src = (size_t)r * LANES + part;  // in 16-byte units
    const size_t dst = (((size_t)page * p.Hkv + h) * p.ps + off) * LANES + part;
    const u32x4_t kv = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p.k) + src);
    const u32x4_t vv = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p.v) + src);
    reinterpret_cast<u32x4_t *>(p.kp)[dst] = kv;
    reinterpret_cast<u32x4_t *>(p.vp)[dst] = vv;
  }
}

template <int LANES>
hipError_t launch(const AppendParams &p, hipStream_t stream) {
  constexpr int kRowsPerBlock = 256 / LANES;
  const long long rows = (long long)p.tokens * p.Hkv;
  const long long want = (rows + kRowsPerBlock - 1) / kRowsPerBlock;
  const int blocks = (int)(want < 256 * 16 ? want : 256 * 16);  // grid-stride past 16 per CU
  hipLaunchKernelGGL((append_kernel<LANES>), dim3(blocks), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_append(const AppendParams &p, hipStream_t stream) {
  if (p.row_bytes == 128) return launch<8>(p, stream);
  if (p.row_bytes == 256) return launch<16>(p, stream);
  return launch<32>(p, stream);
}

}  // namespace pa
