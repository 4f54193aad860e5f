// hbm_probe.hip - a measurement of the read bandwidth the chip actually
// reaches (a ceiling for the weight stream), not part of the product path.
//
// Each workgroup of 512 threads reads one contiguous share of the buffer with
// 16-byte nontemporal loads, eight in flight per thread, and folds every word
// into an XOR that it writes out (so no load can be dropped). This is the
// access pattern of the weight stream without its arithmetic: every byte
// read once, from HBM, in large contiguous runs per compute unit.
#include "mk_q4k.h"
#include "q4k_device.h"
#include "q4k_host.h"

namespace mk {
namespace {

constexpr int PROBE_THREADS = 512;
constexpr int PROBE_DEPTH = 8;

__global__ void __launch_bounds__(PROBE_THREADS)
    hbm_read_kernel(const u32x4* __restrict__ p, size_t n, uint32_t* __restrict__ out) {
  const size_t per = n / gridDim.x;
  const size_t begin = per * blockIdx.x;
  const size_t end = blockIdx.x + 1 == gridDim.x ? n : begin + per;
  const u32x4* q = p + begin;
  const size_t len = end - begin;
  uint32_t acc = 0;
  size_t i = threadIdx.x;
  for (; i + (PROBE_DEPTH - 1) * PROBE_THREADS < len; i += PROBE_DEPTH * PROBE_THREADS) {
    u32x4 v[PROBE_DEPTH];
#pragma unroll
    for (int j = 0; j < PROBE_DEPTH; ++j) v[j] = __builtin_nontemporal_load(q + i + j * PROBE_THREADS);
#pragma unroll
    for (int j = 0; j < PROBE_DEPTH; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
  }
  for (; i < len; i += PROBE_THREADS) {
    const u32x4 v = __builtin_nontemporal_load(q + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  // one word per workgroup: the XOR of its threads' words
  __shared__ uint32_t red[PROBE_THREADS / 64];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t x = 0;
#pragma unroll
    for (int w = 0; w < PROBE_THREADS / 64; ++w) x ^= red[w];
    out[blockIdx.x] = x;
  }
}

}  // namespace
}  // namespace mk

extern "C" int mk_hbm_read_probe(const void* buf, size_t bytes, uint32_t* out, int grid,
                                 void* stream) {
  if (!buf || !out || bytes < 16 || grid < 1 || grid > 65535) return MK_EINVAL;
  if ((reinterpret_cast<uintptr_t>(buf) & 15u) != 0) return MK_EALIGN;
  int cus = 0;
  const int rc = mk::current_gfx950(&cus);
  if (rc != MK_OK) return rc;
  hipLaunchKernelGGL(mk::hbm_read_kernel, dim3(grid), dim3(mk::PROBE_THREADS), 0,
                     static_cast<hipStream_t>(stream), static_cast<const mk::u32x4*>(buf), bytes / 16,
                     out);
  return hipGetLastError() == hipSuccess ? MK_OK : MK_EHIP;
}
