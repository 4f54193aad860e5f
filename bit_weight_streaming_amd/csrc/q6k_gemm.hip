// q6k_gemm.hip - Q6_K weights times M <= 32 stacked binary16 rows.
//
// Q6_K is the other k-quant of Q4_K_M model files (GGUF type 14): 256
// weights in 210 bytes, ql[128] low nibbles, qh[64] high bit pairs, int8
// scales per run of 16 weights, binary16 d. Weight k of a block (half
// h = k / 128, quarter j = (k % 128) / 32, place l = k % 32) has low bits
// nibble j / 2 of ql[64h + 32 (j % 2) + l], high bits 2j..2j+1 of
// qh[32h + l], q = low | high << 4 and value d * sc[k / 16] * (q - 32).
//
// Load-time repack (mk_q6k_repack): 16 rows x one block form a 3360-byte
// tile record laid out for the MFMA lanes. Lane l = 16 g + c (row c of the
// tile, lane group g) feeds, for every run r of the block (one 16x16x16
// MFMA per run), the 4 weights at places 16 (r % 2) + 4 g .. +3 of quarter
// (r % 8) / 2 of half r / 8; its low-nibble bytes are 8 pieces of 4 bytes
// (half h, quarter parity, run parity) and its high-bit bytes 4 pieces
// (half, run parity):
//   bytes    0..2047  lane l's 32 low-nibble bytes at 32 l
//   bytes 2048..3071  lane l's 16 high-bit bytes at 2048 + 16 l
//   bytes 3072..3327  row c's 16 scales at 3072 + 16 c
//   bytes 3328..3359  row c's d at 3328 + 2 c
// Rows past N are zero. Records run tile-major: tile t, block b at
// (t * K/256 + b) * 3360.
//
// Product: D = X W^T per run on v_mfma_f32_16x16x16_f16 (A = 16 rows of X,
// B = the tile's 16 weight rows as exact binary16 q - 32), so lane (c, g)
// holds output column n = c and rows 4g..4g+3 and adds d[n] * sc[n][r]
// times its 4 results in fp32. One workgroup of 8 waves per tile; wave w
// takes blocks w, w + 8, ...; the waves merge in LDS in a fixed order.
#include <string.h>

#include "mk_q4k.h"
#include "mk_q6k.h"
#include "q4k_device.h"

namespace mk {

namespace {

constexpr int Q6_QK = 256;
constexpr int Q6_BLOCK = 210;
constexpr int Q6_REC = 3360;  // 16 rows x 210 bytes
constexpr int Q6_WAVES = 8;
constexpr int Q6_THREADS = 64 * Q6_WAVES;

// Source byte (within a raw 210-byte block) and row of record byte o.
__device__ __forceinline__ void q6_rec_source(int o, int& row, int& src) {
  if (o < 2048) {
    const int l = o >> 5, p = (o & 31) >> 2, e = o & 3;
    const int c = l & 15, g = l >> 4, h = p >> 2, jj = (p >> 1) & 1, rr = p & 1;
    row = c;
    src = 64 * h + 32 * jj + 16 * rr + 4 * g + e;
  } else if (o < 3072) {
    const int o2 = o - 2048, l = o2 >> 4, p = (o2 & 15) >> 2, e = o2 & 3;
    const int c = l & 15, g = l >> 4, h = p >> 1, rr = p & 1;
    row = c;
    src = 128 + 32 * h + 16 * rr + 4 * g + e;
  } else if (o < 3328) {
    row = (o - 3072) >> 4;
    src = 192 + ((o - 3072) & 15);
  } else {
    row = (o - 3328) >> 1;
    src = 208 + ((o - 3328) & 1);
  }
}

// One thread per record byte.
__global__ void __launch_bounds__(256) q6k_repack_kernel(const uint8_t* __restrict__ W,
                                                         uint8_t* __restrict__ T, int N, int nkb,
                                                         long long total) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const long long rec = i / Q6_REC;
  const int o = (int)(i - rec * Q6_REC);
  const int t = (int)(rec / nkb), kb = (int)(rec - (long long)t * nkb);
  int row, src;
  q6_rec_source(o, row, src);
  const int n = 16 * t + row;
  T[i] = n < N ? W[((size_t)n * nkb + kb) * Q6_BLOCK + src] : (uint8_t)0;
}

// Four bytes 0..63 as exact binary16 q - 32 (0x6400 | q is 1024 + q).
__device__ __forceinline__ half4v q6_to_h4(uint32_t q) {
  const u32x2 b = {__builtin_amdgcn_perm(0x64646464u, q, 0x04010400u),
                   __builtin_amdgcn_perm(0x64646464u, q, 0x04030402u)};
  const _Float16 k = (_Float16)1056.f;
  return __builtin_bit_cast(half4v, b) - half4v{k, k, k, k};
}

// ---- Q6_K matrices for the decode-step walk (record layout in q4k_device.h)

// Low 4 and high 2 bits of weight k of a raw 210-byte Q6_K block.
__device__ __forceinline__ int q6_low4(const uint8_t* blk, int k) {
  const int h = k >> 7, j = (k & 127) >> 5, l = k & 31;
  return (blk[64 * h + 32 * (j & 1) + l] >> (4 * (j >> 1))) & 15;
}
__device__ __forceinline__ int q6_high2(const uint8_t* blk, int k) {
  const int h = k >> 7, j = (k & 127) >> 5, l = k & 31;
  return (blk[128 + 32 * h + l] >> (2 * j)) & 3;
}

// One thread per (record, lane): the lane's 16 + 16 + 16 + 4 bytes, and the
// row's d for lanes 0..15. Rows past N are zero.
__global__ void __launch_bounds__(256) q6k_step_repack_kernel(const uint8_t* __restrict__ W,
                                                              uint8_t* __restrict__ T, int N,
                                                              int nkb, long long nthreads) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= nthreads) return;
  const long long rec = i >> 6;
  const int l = (int)(i & 63), c = l & 15, g = l >> 4;
  const int t = (int)(rec / nkb), kb = (int)(rec - (long long)t * nkb);
  const int n = 16 * t + c;
  uint8_t* out = T + rec * Q6W_REC;
  uint8_t qa[16], qb[16], hb[16], sc[4];
  uint16_t d = 0;
  if (n < N) {
    const uint8_t* blk = W + ((size_t)n * nkb + kb) * Q6_BLOCK;
    const int k0 = 64 * g;
    for (int b = 0; b < 16; ++b) {
      qa[b] = (uint8_t)(q6_low4(blk, k0 + b) | (q6_low4(blk, k0 + 32 + b) << 4));
      qb[b] = (uint8_t)(q6_low4(blk, k0 + 16 + b) | (q6_low4(blk, k0 + 48 + b) << 4));
    }
    for (int m = 0; m < 4; ++m)
      for (int b = 0; b < 4; ++b)
        hb[4 * m + b] = (uint8_t)(q6_high2(blk, k0 + 8 * m + b) |
                                  (q6_high2(blk, k0 + 32 + 8 * m + b) << 2) |
                                  (q6_high2(blk, k0 + 8 * m + 4 + b) << 4) |
                                  (q6_high2(blk, k0 + 36 + 8 * m + b) << 6));
    for (int r = 0; r < 4; ++r) sc[r] = blk[192 + 4 * g + r];
    d = (uint16_t)(blk[208] | (blk[209] << 8));
  } else {
    for (int b = 0; b < 16; ++b) qa[b] = qb[b] = hb[b] = 0;
    for (int r = 0; r < 4; ++r) sc[r] = 0;
  }
  for (int b = 0; b < 16; ++b) {
    out[16 * l + b] = qa[b];
    out[1024 + 16 * l + b] = qb[b];
    out[2048 + 16 * l + b] = hb[b];
  }
  for (int r = 0; r < 4; ++r) out[3072 + 4 * l + r] = sc[r];
  if (g == 0) {
    out[3328 + 2 * c] = (uint8_t)(d & 0xFF);
    out[3329 + 2 * c] = (uint8_t)(d >> 8);
  }
}

// Column sums sum_k w[n][k] of the rows of a Q6_K matrix (zero for the rows
// that pad the last tile), one thread per row: per block d * sum_r sc[r] *
// (integer sum of the run's q - 32), exact, added in double; rounded once.
__global__ void __launch_bounds__(256) q6k_colsum_kernel(const uint8_t* __restrict__ W,
                                                         float* __restrict__ cs, int N, int Npad,
                                                         int nkb) {
  const int n = blockIdx.x * blockDim.x + threadIdx.x;
  if (n >= Npad) return;
  double acc = 0.0;
  if (n < N) {
    for (int kb = 0; kb < nkb; ++kb) {
      const uint8_t* blk = W + ((size_t)n * nkb + kb) * Q6_BLOCK;
      long long s = 0;
      for (int r = 0; r < 16; ++r) {
        int qs = 0;
        for (int i = 0; i < 16; ++i) {
          const int k = 16 * r + i;
          qs += (q6_low4(blk, k) | (q6_high2(blk, k) << 4)) - 32;
        }
        s += (long long)(int8_t)blk[192 + r] * qs;
      }
      acc += (double)bit_cast_<_Float16>((uint16_t)(blk[208] | (blk[209] << 8))) * (double)s;
    }
  }
  cs[n] = (float)acc;
}

template <int MT, int TN>
__global__ void __launch_bounds__(Q6_THREADS) q6k_gemm_kernel(const uint8_t* __restrict__ T,
                                                              const uint16_t* __restrict__ X,
                                                              float* __restrict__ Y, int M, int N,
                                                              int K) {
  __shared__ floatx4 red[Q6_WAVES][TN * MT][64];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 15, g = lane >> 4;
  const int t0 = blockIdx.x * TN, nkb = K / Q6_QK;
  const int n_tiles = (N + 15) / 16;

  floatx4 acc[TN][MT];
#pragma unroll
  for (int tn = 0; tn < TN; ++tn)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[tn][mt] = floatx4{0.f, 0.f, 0.f, 0.f};
  // A operand rows: m = 16 mt + c (zeros past M)
  const uint16_t* xr[MT];
  bool live[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    live[mt] = 16 * mt + c < M;
    xr[mt] = X + (size_t)(live[mt] ? 16 * mt + c : 0) * K + 4 * g;
  }

  for (int kb = wave; kb < nkb; kb += Q6_WAVES) {
    // this block's activations: one base per row tile, the runs at constant
    // offsets from it; loaded once for the TN weight tiles
    u32x2 xv[MT][16];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const uint16_t* xb = xr[mt] + (size_t)kb * Q6_QK;
#pragma unroll
      for (int r = 0; r < 16; ++r)
        xv[mt][r] = live[mt] ? *reinterpret_cast<const u32x2*>(xb + 16 * r) : u32x2{0u, 0u};
    }
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) {
      const int t = min(t0 + tn, n_tiles - 1);  // a missing last tile reads the one before
      const uint8_t* rec = T + ((size_t)t * nkb + kb) * Q6_REC;
      const u32x4 ql0 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(rec + 32 * lane));
      const u32x4 ql1 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(rec + 32 * lane + 16));
      const u32x4 qh = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(rec + 2048 + 16 * lane));
      const u32x4 sc = *reinterpret_cast<const u32x4*>(rec + 3072 + 16 * c);
      const uint32_t dw = *reinterpret_cast<const uint32_t*>(rec + 3328 + 4 * (c >> 1));
      const float d = (float)bit_cast_<_Float16>((uint16_t)(dw >> (16 * (c & 1))));
      const uint32_t qlp[8] = {ql0.x, ql0.y, ql0.z, ql0.w, ql1.x, ql1.y, ql1.z, ql1.w};
      const uint32_t qhp[4] = {qh.x, qh.y, qh.z, qh.w};
      const uint32_t scw[4] = {sc.x, sc.y, sc.z, sc.w};
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int h = r >> 3, j = (r & 7) >> 1, rr = r & 1;
        const uint32_t low = (qlp[4 * h + 2 * (j & 1) + rr] >> (4 * (j >> 1))) & 0x0F0F0F0Fu;
        const uint32_t high = ((qhp[2 * h + rr] >> (2 * j)) & 0x03030303u) << 4;
        const half4v wb = q6_to_h4(low | high);
        const float s = d * (float)(int8_t)(scw[r >> 2] >> (8 * (r & 3)));
        const floatx4 ss = {s, s, s, s};
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const floatx4 p = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(half4v, xv[mt][r]), wb,
                                                                   floatx4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
          acc[tn][mt] = __builtin_elementwise_fma(ss, p, acc[tn][mt]);
        }
      }
    }
  }

  // the waves' partial sums, added in wave order
#pragma unroll
  for (int tn = 0; tn < TN; ++tn)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) red[wave][tn * MT + mt][lane] = acc[tn][mt];
  __syncthreads();
  if (wave < TN * MT) {  // wave tn * MT + mt finishes weight tile tn, row tile mt
    const int tn = wave / MT, mt = wave % MT;
    floatx4 o = red[0][wave][lane];
#pragma unroll
    for (int w = 1; w < Q6_WAVES; ++w) o += red[w][wave][lane];
    const int n = 16 * (t0 + tn) + c;
    if (n < N) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 16 * mt + 4 * g + i;
        if (m < M) Y[(size_t)m * N + n] = o[i];
      }
    }
  }
}

bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

}  // namespace mk

namespace mk {
namespace {

// One launch for M <= 32 rows.
int launch_q6(const uint8_t* T, const uint16_t* X, float* Y, int M, int N, int K, hipStream_t st) {
  const int n_tiles = (N + 15) / 16;
  // several weight tiles per workgroup share the activation loads: four
  // where that still leaves 256 workgroups (one row tile), two where it
  // leaves 512; the choice depends on N and the row-tile count only
  const bool pair = (n_tiles + 1) / 2 >= 512;
  const bool quad = (n_tiles + 3) / 4 >= 256;
  const dim3 grid((unsigned)(quad && M <= 16 ? (n_tiles + 3) / 4 : pair ? (n_tiles + 1) / 2 : n_tiles)),
      block(Q6_THREADS);
  if (M <= 16) {
    if (quad)
      hipLaunchKernelGGL((q6k_gemm_kernel<1, 4>), grid, block, 0, st, T, X, Y, M, N, K);
    else if (pair)
      hipLaunchKernelGGL((q6k_gemm_kernel<1, 2>), grid, block, 0, st, T, X, Y, M, N, K);
    else
      hipLaunchKernelGGL((q6k_gemm_kernel<1, 1>), grid, block, 0, st, T, X, Y, M, N, K);
  } else {
    if (pair)
      hipLaunchKernelGGL((q6k_gemm_kernel<2, 2>), grid, block, 0, st, T, X, Y, M, N, K);
    else
      hipLaunchKernelGGL((q6k_gemm_kernel<2, 1>), grid, block, 0, st, T, X, Y, M, N, K);
  }
  return hipGetLastError() == hipSuccess ? MK_OK : MK_EHIP;
}

}  // namespace
}  // namespace mk

extern "C" {

size_t mk_q6k_tiles_bytes(int N, int K) {
  if (N < 1 || K < mk::Q6_QK || K % mk::Q6_QK) return 0;
  return (size_t)((N + 15) / 16) * (K / mk::Q6_QK) * mk::Q6_REC;
}

int mk_q6k_repack(const void* W, void* tiles, int N, int K, void* stream) {
  using namespace mk;
  if (!W || !tiles || N < 1 || K < Q6_QK || K % Q6_QK) return MK_EINVAL;
  if (!al16(tiles)) return MK_EALIGN;
  const long long total = (long long)mk_q6k_tiles_bytes(N, K);
  const long long blocks = (total + 255) / 256;
  if (blocks > 0x7FFFFFFF) return MK_EINVAL;
  hipLaunchKernelGGL(q6k_repack_kernel, dim3((unsigned)blocks), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint8_t*>(W),
                     static_cast<uint8_t*>(tiles), N, K / Q6_QK, total);
  return hipGetLastError() == hipSuccess ? MK_OK : MK_EHIP;
}

int mk_q6k_gemm_tiled(const void* tiles, const uint16_t* X, float* Y, int M, int N, int K,
                      void* stream) {
  using namespace mk;
  if (!tiles || !X || !Y || M < 1 || M > 64 || N < 1 || K < Q6_QK || K % Q6_QK) return MK_EINVAL;
  if (!al16(tiles) || !al16(X) || !al16(Y)) return MK_EALIGN;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const uint8_t* T = static_cast<const uint8_t*>(tiles);
  // up to 32 rows per launch (two row tiles: more spill registers); rows 32..
  // in a second launch over the same weights. A row's result does not depend
  // on the rows beside it, so the split changes no bits.
  for (int r0 = 0; r0 < M; r0 += 32) {
    const int m = M - r0 < 32 ? M - r0 : 32;
    const int rc = launch_q6(T, X + (size_t)r0 * K, Y + (size_t)r0 * N, m, N, K, st);
    if (rc != MK_OK) return rc;
  }
  return MK_OK;
}

size_t mk_q6k_step_bytes(int N, int K) {
  if (N < 1 || K < mk::Q6_QK || K % mk::Q6_QK) return 0;
  const size_t nt = (size_t)((N + 15) / 16);
  return nt * (K / mk::Q6_QK) * mk::Q6W_REC + nt * 16 * sizeof(float);
}

int mk_q6k_step_repack(const void* W, void* out, int N, int K, void* stream) {
  using namespace mk;
  if (!W || !out || N < 1 || K < Q6_QK || K % Q6_QK) return MK_EINVAL;
  if (!al16(out)) return MK_EALIGN;
  const size_t nt = (size_t)((N + 15) / 16);
  const size_t rec_bytes = nt * (K / Q6_QK) * Q6W_REC;
  const size_t in = (size_t)N * (K / Q6_QK) * Q6_BLOCK;
  const char* a = static_cast<const char*>(W);
  const char* b = static_cast<const char*>(out);
  if (a < b + mk_q6k_step_bytes(N, K) && b < a + in) return MK_EINVAL;  // must not overlap
  const long long nthreads = (long long)(rec_bytes / Q6W_REC) * 64;
  const long long blocks = (nthreads + 255) / 256;
  if (blocks > 0x7FFFFFFF) return MK_EINVAL;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(q6k_step_repack_kernel, dim3((unsigned)blocks), dim3(256), 0, st,
                     static_cast<const uint8_t*>(W), static_cast<uint8_t*>(out), N, K / Q6_QK,
                     nthreads);
  if (hipGetLastError() != hipSuccess) return MK_EHIP;
  const int npad = (int)(nt * 16);
  hipLaunchKernelGGL(q6k_colsum_kernel, dim3((unsigned)((npad + 255) / 256)), dim3(256), 0, st,
                     static_cast<const uint8_t*>(W),
                     reinterpret_cast<float*>(static_cast<uint8_t*>(out) + rec_bytes), N, npad,
                     K / Q6_QK);
  return hipGetLastError() == hipSuccess ? MK_OK : MK_EHIP;
}

}  // extern "C"
