// mk_api.hip - the C ABI (include/mk_q4k.h): argument validation, device
// checks, workspace handling and dispatch to the kernels. Validation happens
// before any HIP call, so every rejected call touches no device.
#include <map>
#include <mutex>
#include <stdio.h>
#include <string.h>
#include <utility>
#include <vector>

#include "mk_q4k.h"
#include "mk_q6k.h"
#include "q4k_host.h"

namespace {

constexpr int kMaxDevices = 64;

// Per-device facts, filled on first use.
struct DevInfo {
  int checked = 0;
  int ok = 0;
  int cus = 0;
  hipDeviceProp_t prop;
};
DevInfo g_dev[kMaxDevices];
std::mutex g_dev_mu;

// Library-owned GEMM workspaces (mk_q4k_gemm and mk_q4k_gemm_tiled without
// a caller workspace), one per (device, stream): calls on one stream are
// ordered by it, so they can share one. A workspace that is outgrown is not
// freed (work queued on its stream may still read it; freeing it safely
// would need a synchronisation): it is kept, unused, until the process ends.
struct OwnedWs {
  void* ptr = nullptr;
  size_t bytes = 0;
};
std::map<std::pair<int, void*>, OwnedWs> g_ws;
std::vector<void*> g_ws_retired;
std::mutex g_ws_mu;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int current_device(int* dev_out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MK_ENODEV;
  std::lock_guard<std::mutex> lk(g_dev_mu);
  DevInfo& d = g_dev[dev];
  if (!d.checked) {
    d.checked = 1;
    if (hipGetDeviceProperties(&d.prop, dev) == hipSuccess &&
        strncmp(d.prop.gcnArchName, "gfx950", 6) == 0) {
      d.ok = 1;
      d.cus = d.prop.multiProcessorCount;
    }
  }
  if (!d.ok) return MK_ENODEV;
  *dev_out = dev;
  return MK_OK;
}

int check_gemm_args(const void* W, const uint16_t* X, const float* Y, int M, int N, int K,
                    int fmt) {
  if (!W || !X || !Y) return MK_EINVAL;
  if (M < 1 || M > MK_Q4K_MAX_M || N < 1 || K < MK_Q4K_QK || K % MK_Q4K_QK) return MK_EINVAL;
  if ((long long)N * (K / MK_Q4K_QK) > (1LL << 40)) return MK_EINVAL;
  if (!aligned16(W) || !aligned16(X) || !aligned16(Y)) return MK_EALIGN;
  // Y must not overlap W or X
  const char* y0 = reinterpret_cast<const char*>(Y);
  const char* y1 = y0 + (size_t)M * N * sizeof(float);
  const char* w0 = static_cast<const char*>(W);
  const size_t tiles_kb = (size_t)((N + 15) / 16) * (K / MK_Q4K_QK);
  const char* w1 = w0 + (fmt == mk::GEMM_Q6W     ? tiles_kb * MK_Q6K_TILE_BYTES
                         : fmt == mk::GEMM_TILES ? tiles_kb * 16 * MK_Q4K_BLOCK_BYTES
                                                 : (size_t)N * (K / MK_Q4K_QK) * MK_Q4K_BLOCK_BYTES);
  const char* x0 = reinterpret_cast<const char*>(X);
  const char* x1 = x0 + (size_t)M * K * sizeof(uint16_t);
  if (y0 < w1 && w0 < y1) return MK_EINVAL;
  if (y0 < x1 && x0 < y1) return MK_EINVAL;
  return MK_OK;
}

}  // namespace

namespace mk {
int current_gfx950(int* cus) {
  int dev;
  int rc = current_device(&dev);
  if (rc == MK_OK && cus) *cus = g_dev[dev].cus;
  return rc;
}
}  // namespace mk

namespace {

// CU count assumed for workspace sizing when no gfx950 device is current.
constexpr int kDefaultCus = 256;

// Library-owned workspace of (the current device, stream) with at least
// `bytes` bytes. Sizes start at 64 MiB (every single-matrix plan of the
// workload fits) and at least double when outgrown, so a stream retires few.
int owned_workspace(int dev, void* stream, size_t bytes, void** out) {
  std::lock_guard<std::mutex> lk(g_ws_mu);
  OwnedWs& o = g_ws[std::make_pair(dev, stream)];
  if (o.bytes < bytes) {
    size_t want = o.bytes ? 2 * o.bytes : ((size_t)64 << 20);
    if (want < bytes) want = bytes;
    void* p = nullptr;
    if (hipMalloc(&p, want) != hipSuccess) return MK_EHIP;
    if (o.ptr) g_ws_retired.push_back(o.ptr);
    o.ptr = p;
    o.bytes = want;
  }
  *out = o.ptr;
  return MK_OK;
}

int run_gemm(int fmt, const void* W, const uint16_t* X, float* Y, int M, int N, int K,
             void* workspace, size_t ws_bytes, void* stream) {
  int rc = check_gemm_args(W, X, Y, M, N, K, fmt);
  if (rc != MK_OK) return rc;
  // a caller workspace is validated before the device is looked at
  int dev = -1;
  const bool have_dev = current_device(&dev) == MK_OK;
  const mk::GemmPlan p = mk::gemm_plan(M, N, K, have_dev ? g_dev[dev].cus : kDefaultCus, fmt);
  if (!p.ok) return MK_EINVAL;
  const bool caller_ws = workspace != nullptr || ws_bytes != 0;
  if (caller_ws && p.ws_bytes > 0) {
    if (!workspace || ws_bytes < p.ws_bytes) return MK_EWORKSPACE;
    if (!aligned16(workspace)) return MK_EALIGN;
  }
  if (!have_dev) return MK_ENODEV;
  void* ws = workspace;
  if (!caller_ws && p.ws_bytes > 0) {
    rc = owned_workspace(dev, stream, p.ws_bytes, &ws);
    if (rc != MK_OK) return rc;
  }
  hipError_t e = mk::gemm_launch(p, fmt, W, X, Y, M, N, K, ws, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MK_OK : MK_EHIP;
}

// ---- the GEMM entry point that allocates nothing (mk_q4k_gemm_noalloc)
//
// Its K-split partial sums live in a file-scope device array, `scratch`,
// which every GPU the library runs on holds (one copy per device, at its own
// address) until the process ends. In host code `scratch` names a host-side
// stand-in, not device memory: the device address of each GPU's copy is
// looked up once per device with hipGetSymbolAddress (with that device
// current) and only that address is ever handed to kernels.
static __device__ __align__(256) char scratch[MK_Q4K_NOALLOC_SCRATCH_BYTES];

struct ScratchAddr {
  int looked_up = 0;
  void* ptr = nullptr;
};
ScratchAddr g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of the current device's copy of `scratch`.
int scratch_address(int dev, void** out) {
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  ScratchAddr& a = g_scratch[dev];
  if (!a.looked_up) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MK_EHIP;
    a.ptr = p;
    a.looked_up = 1;
  }
  *out = a.ptr;
  return MK_OK;
}

}  // namespace

extern "C" {

int mk_q4k_gemm_noalloc(const void* W_blocks, const uint16_t* X_fp16, float* Y_fp32, int M, int N,
                        int K, void* stream) {
  int rc = check_gemm_args(W_blocks, X_fp16, Y_fp32, M, N, K, mk::GEMM_ROWS);
  if (rc != MK_OK) return rc;
  int dev = -1;
  rc = current_device(&dev);
  if (rc != MK_OK) return rc;
  const mk::GemmPlan p = mk::gemm_plan(M, N, K, g_dev[dev].cus);
  if (!p.ok) return MK_EINVAL;
  if (p.ws_bytes > (size_t)MK_Q4K_NOALLOC_SCRATCH_BYTES) return MK_EWORKSPACE;
  void* ws = nullptr;
  if (p.ws_bytes > 0) {
    rc = scratch_address(dev, &ws);
    if (rc != MK_OK) return rc;
  }
  hipError_t e =
      mk::gemm_launch(p, false, W_blocks, X_fp16, Y_fp32, M, N, K, ws, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MK_OK : MK_EHIP;
}

const char* mk_strerror(int code) {
  switch (code) {
    case MK_OK: return "ok";
    case MK_EINVAL: return "invalid argument (shape, null pointer, overlap or layer chain)";
    case MK_EALIGN: return "pointer not 16-byte aligned";
    case MK_EWORKSPACE: return "workspace missing or too small";
    case MK_EOCCUPANCY: return "persistent grid cannot be co-resident on this device";
    case MK_EHIP: return "HIP runtime error";
    case MK_ENODEV: return "current device is not a gfx950 GPU";
    case MK_ETIMEOUT: return "device: grid barrier wait timed out";
    case MK_ERANGE: return "device: row statistic out of representable range";
    default: return "unknown error code";
  }
}

int mk_device_info(char* buf, size_t len) {
  if (!buf || len == 0) return MK_EINVAL;
  int dev;
  int rc = current_device(&dev);
  if (rc != MK_OK) {
    snprintf(buf, len, "no gfx950 device");
    return rc;
  }
  const hipDeviceProp_t& p = g_dev[dev].prop;
  snprintf(buf, len,
           "{\"name\": \"%s\", \"arch\": \"%s\", \"cus\": %d, \"lds_per_block\": %zu, "
           "\"clock_khz\": %d, \"mem_clock_khz\": %d, \"bus_bits\": %d, \"l2_bytes\": %d, "
           "\"hbm_bytes\": %zu}",
           p.name, p.gcnArchName, p.multiProcessorCount, (size_t)p.sharedMemPerBlock, p.clockRate,
           p.memoryClockRate, p.memoryBusWidth, p.l2CacheSize, (size_t)p.totalGlobalMem);
  return MK_OK;
}

size_t mk_q4k_gemm_workspace_bytes(int M, int N, int K) {
  if (M < 1 || M > MK_Q4K_MAX_M || N < 1 || K < MK_Q4K_QK || K % MK_Q4K_QK) return 0;
  int cus = 0;
  if (mk::current_gfx950(&cus) != MK_OK) cus = kDefaultCus;
  return mk::gemm_plan(M, N, K, cus).ws_bytes;
}

int mk_q4k_gemm_ws(const void* W_blocks, const uint16_t* X_fp16, float* Y_fp32, int M, int N,
                   int K, void* workspace, size_t ws_bytes, void* stream) {
  return run_gemm(mk::GEMM_ROWS, W_blocks, X_fp16, Y_fp32, M, N, K, workspace, ws_bytes, stream);
}

int mk_q4k_gemm(const void* W_blocks, const uint16_t* X_fp16, float* Y_fp32, int M, int N, int K,
                void* stream) {
  return run_gemm(mk::GEMM_ROWS, W_blocks, X_fp16, Y_fp32, M, N, K, nullptr, 0, stream);
}

int mk_q4k_gemm_tiled(const void* W_tiles, const uint16_t* X_fp16, float* Y_fp32, int M, int N,
                      int K, void* stream) {
  return run_gemm(mk::GEMM_TILES, W_tiles, X_fp16, Y_fp32, M, N, K, nullptr, 0, stream);
}

int mk_q6k_gemm_step(const void* W_step, const uint16_t* X_fp16, float* Y_fp32, int M, int N,
                     int K, void* stream) {
  return run_gemm(mk::GEMM_Q6W, W_step, X_fp16, Y_fp32, M, N, K, nullptr, 0, stream);
}

}  // extern "C"
