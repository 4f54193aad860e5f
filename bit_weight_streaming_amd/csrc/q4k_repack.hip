// q4k_repack.hip - load-time reordering of Q4_K rows into the 16-row tile
// records the streaming kernels read, followed by the weights' column sums.
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

// Column sums of the weights, sum_k w[n][k] for every row n of W (zero for
// the rows that pad the last tile), rounded once to fp32. One thread per row
// adds its blocks in order in double precision; within a block the sum is
// d * sum_j sc_j * Q_j - dmin * 32 * sum_j m_j with Q_j the integer sum of the
// 32 quants of sub-block j, so each block's term is exact.
__global__ void __launch_bounds__(256)
    q4k_colsum_kernel(const uint8_t* __restrict__ src, float* __restrict__ cs, int N, int Npad,
                      int KB) {
  const int n = blockIdx.x * blockDim.x + threadIdx.x;
  if (n >= Npad) return;
  double acc = 0.0;
  if (n < N) {
    for (int kb = 0; kb < KB; ++kb) {
      const uint8_t* b = src + ((size_t)n * KB + kb) * BLOCK_BYTES;
      const _Float16 d = bit_cast_<_Float16>((uint16_t)(b[0] | (b[1] << 8)));
      const _Float16 dmin = bit_cast_<_Float16>((uint16_t)(b[2] | (b[3] << 8)));
      const uint8_t* s = b + 4;
      long long scq = 0, msum = 0;
      for (int j = 0; j < 8; ++j) {
        int sc, m;
        if (j < 4) {
          sc = s[j] & 63;
          m = s[j + 4] & 63;
        } else {
          sc = (s[j + 4] & 15) | ((s[j - 4] >> 6) << 4);
          m = (s[j + 4] >> 4) | ((s[j] >> 6) << 4);
        }
        // quants of sub-block j: chunk j/2, low nibbles for even j
        const uint8_t* q = b + 16 + 32 * (j >> 1);
        int qs = 0;
        for (int i = 0; i < 32; ++i) qs += (j & 1) ? (q[i] >> 4) : (q[i] & 15);
        scq += (long long)sc * qs;
        msum += m;
      }
      acc += (double)d * (double)scq - (double)dmin * (double)(32 * msum);
    }
  }
  cs[n] = (float)acc;
}

}  // namespace mk

extern "C" {

size_t mk_q4k_tiles_bytes(int N, int K) {
  if (N < 1 || K < MK_Q4K_QK || K % MK_Q4K_QK) return 0;
  const size_t nt = (size_t)((N + 15) / 16);
  return nt * (K / MK_Q4K_QK) * mk::TILE_RECORD_BYTES + nt * 16 * sizeof(float);
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
  const size_t nt = (size_t)((N + 15) / 16);
  const size_t rec_bytes = nt * (K / MK_Q4K_QK) * mk::TILE_RECORD_BYTES;
  const long long nchunks = (long long)(rec_bytes / 16);
  long long blocks = (nchunks + 255) / 256;
  if (blocks > 16384) blocks = 16384;
  hipLaunchKernelGGL(mk::q4k_repack_kernel, dim3((unsigned)blocks), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint8_t*>(W_rows),
                     static_cast<uint8_t*>(W_tiles), N, K / MK_Q4K_QK, nchunks);
  if (hipGetLastError() != hipSuccess) return MK_EHIP;
  const int npad = (int)(nt * 16);
  hipLaunchKernelGGL(mk::q4k_colsum_kernel, dim3((unsigned)((npad + 255) / 256)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint8_t*>(W_rows),
                     reinterpret_cast<float*>(static_cast<uint8_t*>(W_tiles) + rec_bytes), N,
                     npad, K / MK_Q4K_QK);
  return hipGetLastError() == hipSuccess ? MK_OK : MK_EHIP;
}

}  // extern "C"
