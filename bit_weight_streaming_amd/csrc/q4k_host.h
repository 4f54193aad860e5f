// q4k_host.h - internal host-side declarations shared by the library's
// translation units (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mk {

// Launch plan of the single-matrix GEMM for one (M, N, K).
struct GemmPlan {
  int mt = 1;          // 16-row MFMA tiles covering M
  int ks = 1;          // K slices (workgroup rows of the grid)
  int nkb = 1;         // super-blocks per slice
  int groups = 1;      // workgroups per slice (4 column tiles each)
  size_t lds = 0;      // dynamic LDS bytes
  size_t ws_bytes = 0; // partial-sum workspace (0 when ks == 1)
};

GemmPlan gemm_plan(int M, int N, int K);
hipError_t gemm_launch(const GemmPlan& p, const void* W, const uint16_t* X, float* Y, int M, int N,
                       int K, void* ws, hipStream_t st);

}  // namespace mk

namespace mk {
// MK_OK and the CU count of the current device if it is a gfx950 GPU,
// MK_ENODEV otherwise.
int current_gfx950(int* cus);
}  // namespace mk
