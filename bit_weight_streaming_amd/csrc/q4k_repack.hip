// q4k_repack.hip - load-time reordering of Q4_K rows into the 16-row tile
// records the streaming kernels read.
//
// The bytes of every block are kept; only their order changes. Rows are cut
// into tiles of 16 (rows past N are zero blocks). For tile t and super-block
// kb the record at ((t * KB) + kb) * 2304 holds
//   [0, 256)     the 16-byte header (d, dmin, 12 scale bytes) of rows 16t+i,
//                i = 0..15
//   [256, 1280)  entry l = i + 16g (l = 0..63): quant bytes [32g, 32g+16) of
//                row 16t+i
//   [1280, 2304) entry l: quant bytes [32g+16, 32g+32) of row 16t+i
// so that lane l of a wave reads its three 16-byte operands of one block with
// wave-wide loads of 256 (broadcast), 1024 and 1024 contiguous bytes.
#include "mk_q4k.h"
#include "q4k_device.h"

namespace mk {

constexpr int TILE_RECORD_BYTES = 16 * BLOCK_BYTES;  // 2304

// One thread per 16-byte chunk of the output (144 chunks per record).
__global__ void __launch_bounds__(256)
    q4k_repack_kernel(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst, int N, int KB,
                      long long nchunks) {
  for (long long c = (long long)blockIdx.x * blockDim.x + threadIdx.x; c < nchunks;
       c += (long long)gridDim.x * blockDim.x) {
    const long long rec = c / 144;
    const int j = (int)(c - rec * 144);
    const long long t = rec / KB;
    const int kb = (int)(rec - t * KB);
    int i, off;
    if (j < 16) {
      i = j;
      off = 0;
    } else if (j < 80) {
      const int l = j - 16;
      i = l & 15;
      off = 16 + 32 * (l >> 4);
    } else {
      const int l = j - 80;
      i = l & 15;
      off = 32 + 32 * (l >> 4);
    }
    const long long row = t * 16 + i;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (row < N) v = *reinterpret_cast<const u32x4*>(src + (row * KB + kb) * BLOCK_BYTES + off);
    *reinterpret_cast<u32x4*>(dst + c * 16) = v;
  }
}

}  // namespace mk

extern "C" {

size_t mk_q4k_tiles_bytes(int N, int K) {
  if (N < 1 || K < MK_Q4K_QK || K % MK_Q4K_QK) return 0;
  return (size_t)((N + 15) / 16) * (K / MK_Q4K_QK) * mk::TILE_RECORD_BYTES;
}

int mk_q4k_repack(const void* W_rows, void* W_tiles, int N, int K, void* stream) {
  if (!W_rows || !W_tiles || N < 1 || K < MK_Q4K_QK || K % MK_Q4K_QK) return MK_EINVAL;
  if ((reinterpret_cast<uintptr_t>(W_rows) & 15) || (reinterpret_cast<uintptr_t>(W_tiles) & 15))
    return MK_EALIGN;
  const size_t out = mk_q4k_tiles_bytes(N, K);
  const size_t in = (size_t)N * (K / MK_Q4K_QK) * MK_Q4K_BLOCK_BYTES;
  const char* a = static_cast<const char*>(W_rows);
  const char* b = static_cast<const char*>(W_tiles);
  if (a < b + out && b < a + in) return MK_EINVAL;  // must not overlap
  const long long nchunks = (long long)(out / 16);
  long long blocks = (nchunks + 255) / 256;
  if (blocks > 16384) blocks = 16384;
  hipLaunchKernelGGL(mk::q4k_repack_kernel, dim3((unsigned)blocks), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint8_t*>(W_rows),
                     static_cast<uint8_t*>(W_tiles), N, K / MK_Q4K_QK, nchunks);
  return hipGetLastError() == hipSuccess ? MK_OK : MK_EHIP;
}

}  // extern "C"
