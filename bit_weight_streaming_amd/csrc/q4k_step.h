// q4k_step.h - host/device shared definitions of the persistent decode-step
// walk (internal; the public interface is mk_q4k_step in mk_q4k.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mk {

constexpr int STEP_WAVES = 8;
constexpr int STEP_THREADS = 64 * STEP_WAVES;
constexpr int STEP_PD = 4;       // weight records in flight per wave (more spills registers)
constexpr int STEP_MAX_LAYERS = 128;
constexpr int STAT_SLOTS = 64;   // spread of the row-statistic atomics
constexpr int DONE_CTRS = 64;    // spread of the finished-tile counters
constexpr int CTR_STRIDE = 32;   // uints between counters (128 bytes)
constexpr int STEP_MAX_M = 16;   // rows one walk takes (one MFMA row tile)
// Rows a step call takes: more than STEP_MAX_M run as consecutive walks over
// row groups of STEP_MAX_M (each row's arithmetic is the same in any group).
constexpr int STEP_MAX_ROWS = 64;
constexpr int STEP_GROUPS = STEP_MAX_ROWS / STEP_MAX_M;

// Build-time option of the walk (a measurement aid, off in the product
// library): with MK_STEP_TIMELINE=1 thread 0 of every workgroup stores the
// wall clock (s_memrealtime, 100 MHz) at five points of each phase of each
// layer into a region of the workspace (TL_EVENTS slots per (layer, phase,
// workgroup)): compute start (input staged), compute end, slice partials
// published, own tiles finished, the phase's done counters seen.
#ifndef MK_STEP_TIMELINE
#define MK_STEP_TIMELINE 0
#endif
constexpr int TL_EVENTS = 8;  // slots per (layer, phase, workgroup); 5 used
enum TlEvent { TL_START = 0, TL_COMPUTED = 1, TL_PUBLISHED = 2, TL_FINISHED = 3, TL_DONE_SEEN = 4 };

// Fixed-point scales of the row statistics of a phase input: sum(x) * 2^24
// (exact for binary16 values) and sum(x^2) * 2^20, accumulated with 64-bit
// integer atomics, so the totals do not depend on the order in which
// workgroups add them. One contribution (a tile row) must stay below 2^50 in
// magnitude, which keeps any total of up to 8192 tiles inside 63 bits.
//
// Each workgroup sums its contributions in LDS and adds its share S to the
// word of its slot (workgroup w: slot w % STAT_SLOTS) as 32 S + 1, after it
// has counted its tiles finished. The low five bits of a word count the
// shares that are in, so a consumer that staged the words before every share
// arrived sees it (all words of a phase input count 2 M G shares when
// complete) and reloads them before it needs the totals. A slot's sum must
// stay below 2^58 in magnitude: at most STAT_SLOT_TERMS contributions of 2^50
// per slot, which the plan checks.
constexpr double STAT_SCALE_SUM = 16777216.0;
constexpr double STAT_SCALE_SQ = 1048576.0;
constexpr double STAT_TERM_MAX = 1125899906842624.0;  // 2^50
constexpr int STAT_CNT_BITS = 5;                      // share count in the low bits
constexpr int STAT_SLOT_TERMS = 255;                  // 255 * 2^50 < 2^58

// A slice partial carries the parity of its layer in the lowest bit of each
// word: the producer sets it, the finisher waits until every word of a piece
// shows the layer's parity and clears the bit before adding (a change of at
// most one unit in the last place of a partial; a zero partial stays zero).
// Every piece of a phase is rewritten in every layer, so a piece still
// holding the previous layer's value always shows the other parity. Before a
// step all pieces are filled with PART_FILL, whose parity is 1 (layer 0
// expects 0).
constexpr uint32_t PART_FILL = 1u;

// One phase of a layer (the same for every layer).
struct DevPhase {
  int K;           // input width
  int KB;          // K / 256
  int nm;          // matrices per tile: 1, or 2 (gate and up paired)
  int nseg;        // column segments (phase A: q | k | v)
  int seg_n[3];    // columns of each segment
  int seg_t0[4];   // first tile of each segment; seg_t0[nseg] = total tiles
  int seg_c0[3];   // first column of each segment in the partial buffer
  int mat0;        // index (0..6) of the first matrix of the phase
  int nt;          // tiles (16 columns each)
  int ncols;       // columns of the partial buffer (gate/up: 2F)
  int sk;          // K slices
  int nkb;         // super-blocks per slice (the last slice may be shorter)
  int x_stride;    // LDS bytes per staged activation row
  int tw_max;      // most tiles one workgroup owns
  int cmax;        // most waves of one workgroup that share a tile
  int lds_contrib; // LDS offset of the per-tile wave contributions
  int lds_bytes;   // LDS this phase needs
  size_t part_off; // workspace offset of the slice partials: one 1 KiB block
                   // (16 x 16 fp32 in MFMA lane order) per (tile, slice, matrix)
  unsigned part_bytes;
  unsigned cs_off[3];  // byte offset of each segment matrix's column sums
                       // in its tile-record buffer (after the records)
  unsigned cs_off6[3]; // the same for a Q6_K matrix (its records are larger)
  double inv_k;        // 1 / K (the row statistics of the input run over K)
  int tab;             // 1: every wave's records fit a record table (the walk's
                       // branch-free loop); 0: the record iterator walks them
  int norm;            // what the products of the phase are scaled by per row:
                       // NORM_STD, NORM_RMS or NORM_NONE
};

// Row scaling of a phase's products. NORM_STD: the standardization of the
// binary16 input, (z - mean * colsum) / sqrt(var + 1e-6), from the sums of x
// and x^2. NORM_RMS (residual walk): z / sqrt(mean(h^2) + 1e-6) of the fp32
// residual h whose normed cast is the input, from the sum of h^2 held as two
// integer words (see RMS_SCALE). NORM_NONE: z itself.
constexpr int NORM_STD = 0, NORM_RMS = 1, NORM_NONE = 2;

// Sum of h^2 in the residual walk: each term (a tile row's fp32 sum of
// squares) is rounded to an integer at scale 2^40 and split at 2^32 into a
// high and a low word, added separately (order independent); the total is
// hi * 2^32 + lo at the same scale. A term must stay below 2^42 (unscaled).
constexpr double RMS_SCALE = 1099511627776.0;     // 2^40
constexpr double RMS_TERM_MAX = 4398046511104.0;  // 2^42

// Device copy of one layer's pointers.
struct DevLayer {
  const uint8_t* w[7];
  float* y[7];
  uint16_t* x[4];
  float* h[2];        // residual walk: fp32 residual after o (h[0]) and after down (h[1])
  const float* g[2];  // residual walk: RMSNorm weights before q/k/v (g[0]) and gate/up (g[1])
  uint32_t q6;        // bit t: matrix t is in the Q6_K walk-record form (v, down only)
  uint32_t pad_;
};

struct StepParams {
  DevPhase ph[4];        // the four phases (kernel arguments: read through the scalar cache)
  int n_layers;
  int M;
  int G;                 // workgroups (one per CU)
  int H;                 // hidden size (x width)
  const uint16_t* x0;
  uint16_t* x_out;
  const float* h0;       // residual walk: fp32 residual entering layer 0
  char* ws;              // workspace base
  size_t layers_off;     // DevLayer table
  size_t done_off;       // DONE_CTRS finished-tile counters
  size_t start_off;      // workgroups done with the layer-0 input statistics
  size_t stats_off;      // [n_layers][4][STAT_SLOTS][M][2] int64: row sums of
                         // the input of phase p of layer l
  size_t status_off;     // int status word
  size_t lds_bytes;
  size_t tl_off;         // MK_STEP_TIMELINE: [n_layers][4][G][TL_EVENTS] u64 stamps
  int reload;            // testing aid: every phase reloads its input statistics at
                         // the end of its compute, as when they were staged incomplete
};

}  // namespace mk
