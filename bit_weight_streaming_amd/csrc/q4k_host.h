// q4k_host.h - internal host-side declarations shared by the library's
// translation units (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mk {

// Launch plan of the single-matrix GEMM for one (M, N, K) on G workgroups.
struct GemmPlan {
  int mt = 1;            // 16-row MFMA tiles covering M
  int KB = 1;            // K / 256
  int nt = 1;            // 16-column tiles covering N
  int G = 1;             // workgroups (one per CU)
  int sk = 1;            // K slices
  int nkb = 1;           // super-blocks per slice (the last may be shorter)
  int x_stride = 0;      // LDS bytes per staged activation row
  size_t lds = 0;        // dynamic LDS bytes
  size_t part_bytes = 0; // slice partials (0 when sk == 1)
  size_t part_off = 0;   // offset of the slice partials in the workspace
  size_t ws_bytes = 0;   // workspace bytes (0 when sk == 1)
  bool ok = false;       // the plan fits the device
};

// Weight forms the single-matrix GEMM reads: Q4_K row blocks, Q4_K tile
// records, Q6_K walk records.
constexpr int GEMM_ROWS = 0, GEMM_TILES = 1, GEMM_Q6W = 2;

GemmPlan gemm_plan(int M, int N, int K, int G, int fmt = GEMM_ROWS);
hipError_t gemm_launch(const GemmPlan& p, int fmt, const void* W, const uint16_t* X, float* Y,
                       int M, int N, int K, void* ws, hipStream_t st);

}  // namespace mk

namespace mk {
// MK_OK and the CU count of the current device if it is a gfx950 GPU,
// MK_ENODEV otherwise.
int current_gfx950(int* cus);
}  // namespace mk
