// q4k_gemm.hip - single-matrix Q4_K weight-streaming GEMM, Y = X * W^T.
//
// Grid: x = groups of WAVES column tiles (16 columns per wave), y = K slices.
// Each workgroup stages the activations of its K slice into LDS once, then
// every wave streams the Q4_K blocks of its 16 weight rows over that slice
// through a register ring of PD blocks in flight, multiplying each block
// against all M rows (mma_block). With one slice the result goes straight to
// Y; with several, each slice writes fp32 partials and a second kernel adds
// them in slice order (deterministic; no floating-point atomics).
#include "q4k_device.h"
#include "q4k_host.h"

namespace mk {

constexpr int GEMM_WAVES = 4;
constexpr int GEMM_THREADS = 64 * GEMM_WAVES;

template <int MT, int PD>
__global__ void __launch_bounds__(GEMM_THREADS)
    q4k_gemm_kernel(const uint8_t* __restrict__ W, const uint16_t* __restrict__ X,
                    float* __restrict__ out, int M, int N, int K, int nkb_slice) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int KB = K / QK;
  const int slice = blockIdx.y;
  const int kb0 = slice * nkb_slice;
  const int nkb = min(nkb_slice, KB - kb0);
  const int row_stride = nkb_slice * X_BYTES_PER_BLOCK + X_ROW_PAD;
  char* x_lds = smem;
  char* xs_lds = smem + (size_t)M * row_stride;

  stage_x(X, K, M, kb0, nkb, x_lds, row_stride, xs_lds, threadIdx.x, GEMM_THREADS);
  __syncthreads();

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int c = lane & 15;   // B/C column within the tile; also the A-operand row
  const int g = lane >> 4;   // quant chunk / k group
  const int col0 = (blockIdx.x * GEMM_WAVES + wave) * 16;
  if (col0 >= N) return;
  // rows past N (ragged last tile) read the last valid row; never stored
  const int col = min(col0 + c, N - 1);
  const uint8_t* wrow = W + ((size_t)col * KB + kb0) * BLOCK_BYTES;

  const char* xa0[MT];
  const char* xs0[MT];
#pragma unroll
  for (int rt = 0; rt < MT; ++rt) {
    const int m = 16 * rt + c;
    xa0[rt] = m < M ? x_lds + (size_t)m * row_stride + g * 128 : nullptr;
    xs0[rt] = m < M ? xs_lds + (size_t)m * nkb * XSUM_BYTES_PER_BLOCK + 8 * g : nullptr;
  }
  floatx4 acc[MT];
#pragma unroll
  for (int rt = 0; rt < MT; ++rt) acc[rt] = floatx4{0.f, 0.f, 0.f, 0.f};

  // Register ring of PD blocks in flight. The steady-state loop issues its
  // loads unconditionally (past the end it re-reads the last block, which is
  // never consumed) so the compiler can wait for exactly the oldest block.
  BlockRegs ring[PD];
#pragma unroll
  for (int s = 0; s < PD; ++s) load_block(ring[s], wrow + (size_t)min(s, nkb - 1) * BLOCK_BYTES, g);

  auto consume = [&](const BlockRegs& r, int b) {
    const char* xa[MT];
    const char* xs[MT];
#pragma unroll
    for (int rt = 0; rt < MT; ++rt) {
      xa[rt] = xa0[rt] ? xa0[rt] + b * X_BYTES_PER_BLOCK : nullptr;
      xs[rt] = xs0[rt] ? xs0[rt] + b * XSUM_BYTES_PER_BLOCK : nullptr;
    }
    mma_block<MT>(r, g, xa, xs, acc);
  };
  int b = 0;
  for (; b + PD <= nkb; b += PD) {
#pragma unroll
    for (int s = 0; s < PD; ++s) {
      consume(ring[s], b + s);
      load_block(ring[s], wrow + (size_t)min(b + s + PD, nkb - 1) * BLOCK_BYTES, g);
    }
  }
#pragma unroll
  for (int s = 0; s < PD; ++s)
    if (b + s < nkb) consume(ring[s], b + s);

  if (col0 + c < N) {
    float* o = out + (size_t)slice * M * N + col0 + c;
#pragma unroll
    for (int rt = 0; rt < MT; ++rt) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = 16 * rt + 4 * g + r;
        if (m < M) o[(size_t)m * N] = acc[rt][r];
      }
    }
  }
}

// Y[i] = sum_s P[s][i] in slice order.
__global__ void __launch_bounds__(256)
    q4k_reduce_slices(const float* __restrict__ P, float* __restrict__ Y, long long n, int ks) {
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (long long)gridDim.x * blockDim.x) {
    float s = P[i];
    for (int k = 1; k < ks; ++k) s += P[(size_t)k * n + i];
    Y[i] = s;
  }
}

GemmPlan gemm_plan(int M, int N, int K) {
  GemmPlan p;
  const int KB = K / QK;
  p.mt = (M + 15) / 16;
  // LDS budget for the staged activations of one slice
  const size_t budget = p.mt >= 4 ? 120 * 1024 : 48 * 1024;
  const size_t per_block = (size_t)M * (X_BYTES_PER_BLOCK + XSUM_BYTES_PER_BLOCK);
  int nkb = (int)((budget - (size_t)M * X_ROW_PAD) / per_block);
  if (nkb < 1) nkb = 1;
  if (nkb > KB) nkb = KB;
  p.ks = (KB + nkb - 1) / nkb;
  p.nkb = (KB + p.ks - 1) / p.ks;  // even out the slices
  p.lds = (size_t)M * (p.nkb * X_BYTES_PER_BLOCK + X_ROW_PAD) +
          (size_t)M * p.nkb * XSUM_BYTES_PER_BLOCK;
  p.groups = ((N + 15) / 16 + GEMM_WAVES - 1) / GEMM_WAVES;
  p.ws_bytes = p.ks > 1 ? (size_t)p.ks * M * N * sizeof(float) : 0;
  return p;
}

template <int MT>
static hipError_t launch_mt(const GemmPlan& p, const uint8_t* W, const uint16_t* X, float* out,
                            int M, int N, int K, hipStream_t st) {
  constexpr int PD = 4;
  auto kern = q4k_gemm_kernel<MT, PD>;
  hipError_t e = hipFuncSetAttribute((const void*)kern,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)p.lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(p.groups, p.ks), dim3(GEMM_THREADS), p.lds, st, W, X, out, M, N,
                     K, p.nkb);
  return hipGetLastError();
}

hipError_t gemm_launch(const GemmPlan& p, const void* W, const uint16_t* X, float* Y, int M, int N,
                       int K, void* ws, hipStream_t st) {
  float* out = p.ks > 1 ? static_cast<float*>(ws) : Y;
  const uint8_t* w = static_cast<const uint8_t*>(W);
  hipError_t e;
  switch (p.mt) {
    case 1: e = launch_mt<1>(p, w, X, out, M, N, K, st); break;
    case 2: e = launch_mt<2>(p, w, X, out, M, N, K, st); break;
    case 3: e = launch_mt<3>(p, w, X, out, M, N, K, st); break;
    default: e = launch_mt<4>(p, w, X, out, M, N, K, st); break;
  }
  if (e != hipSuccess || p.ks == 1) return e;
  const long long n = (long long)M * N;
  int blocks = (int)((n + 255) / 256);
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(q4k_reduce_slices, dim3(blocks), dim3(256), 0, st, out, Y, n, p.ks);
  return hipGetLastError();
}

}  // namespace mk
