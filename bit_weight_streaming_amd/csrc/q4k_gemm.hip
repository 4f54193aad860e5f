// q4k_gemm.hip - single-matrix Q4_K weight-streaming GEMM, Y = X * W^T.
//
// One persistent pass over the weights (the multi-row decode step of the
// OpenJet post, "RTX 3090 one card, four coding agents", paragraph on how
// parallel decoding works: each weight is read once and multiplied against
// every stacked row while on chip).
//
// Grid: one workgroup per CU, 8 waves. The K range is cut into sk slices; the
// workgroups are spread over the slices (assign_split) and each stages the M
// activation rows of its slice into LDS once. The workgroup's (16-column
// tile, super-block) units are split over its waves; every wave streams its
// units through a register ring (GemmRing) and multiplies each record
// against all M rows (MT 16-row MFMA tiles). A tile that one wave computes
// alone is written straight out: to Y when there is one K slice, as a slice
// partial otherwise. A wave keeps its parts of the (at most two) tiles it
// shares with other waves in registers until the stream ends; they are then
// written to LDS over the staged activations and added in wave order. With
// several slices a second kernel on the same stream adds each tile's sk
// partials in slice order and writes Y: no workgroup ever waits for another
// one, no counters are kept between calls, and no floating-point atomics are
// used.
//
// FMT selects the weights' form: GEMM_ROWS, the plain Q4_K row layout read in
// place; GEMM_TILES, the load-time Q4_K tile records (mk_q4k_repack: every
// wave load is one contiguous 1 KiB piece); GEMM_Q6W, Q6_K matrices in the
// decode step's walk records (mk_q6k_step_repack: 3360 bytes per 16 rows and
// block, streamed through the same ring with the lane's run scales).
#include <map>
#include <mutex>
#include <tuple>
#include <utility>

#include "mk_q4k.h"
#include "q4k_device.h"
#include "q4k_host.h"

namespace mk {

constexpr int GEMM_THREADS = 64 * SPLIT_WAVES;
constexpr size_t kGemmLdsLimit = 160 * 1024;

struct GemmArgs {
  const uint8_t* w;    // weights: tile records (TILED) or row blocks
  const uint16_t* x;   // [M][K] binary16
  float* y;            // [M][N]
  char* part;          // slice partials
  unsigned part_bytes; // bytes of slice partials
  int M, N, K, KB, nt, sk, nkb, G, x_stride;
};

template <int MT>
struct GemmRing {  // records in flight per wave (4: six were slower at one row tile)
  static constexpr int PD = 4;
};

template <int MT, int FMT>
__global__ void __launch_bounds__(GEMM_THREADS) q4k_gemm_kernel(GemmArgs A) {
  constexpr bool Q6 = FMT == GEMM_Q6W;
  constexpr int PD = GemmRing<MT>::PD;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int tid = threadIdx.x;
  const int wave = uni(tid >> 6), lane = tid & 63, c = lane & 15, g = lane >> 4;
  const Assign a = assign_split(A.nt, A.sk, A.nkb, A.KB, blockIdx.x, A.G);
  char* x_lds = smem;
  char* xs_lds = smem + (size_t)A.M * A.x_stride;
  // the wave parts of shared tiles are written once the stream has ended,
  // over the staged activations
  char* contrib = smem;

  // this lane's activations of each row tile (rows past M read row M-1; their
  // results are never stored, so every read is unconditional)
  const char* xa[MT];
  const char* xs[MT];
#pragma unroll
  for (int rt = 0; rt < MT; ++rt) {
    const int row = min(16 * rt + c, A.M - 1);
    xa[rt] = x_lds + (size_t)row * A.x_stride + g * 128;
    xs[rt] = xs_lds + (size_t)row * xsum_row_bytes(a.nkb) + 16 * g;
  }
  const UnpackConsts k = unpack_consts(g);
  const __amdgpu_buffer_rsrc_t pr = make_rsrc(A.part, A.part_bytes);

  // the result of tile tg, row tile rt, lane ln: to Y, or as this slice's partial
  auto put = [&](int tg, int ln, const floatx4& v, int rt) {
    if (A.sk == 1) {
      const int col = 16 * tg + (ln & 15);
      if (col < A.N) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = 16 * rt + 4 * (ln >> 4) + r;
          if (m < A.M) A.y[(size_t)m * A.N + col] = v[r];
        }
      }
    } else {
      st4_dev(pr, ((unsigned)(tg * A.sk + a.s) * MT + rt) * 1024u + ln * 16, v);
    }
  };
  // LDS slot of wave v: 0 = the tile that began before its range, 1 = the
  // tile that goes on after it
  auto slot = [&](int v, int ab, int rt) -> char* {
    return contrib + ((size_t)(v * 2 + ab) * MT + rt) * 1024;
  };

  const int ua = wave_begin(a, wave), ub = wave_begin(a, wave + 1);
  // next unit to load (the loop below never asks for one past ub)
  int ltl = ua / a.nkb, lb = ua - ltl * a.nkb, lu = ua;
  BlockRegs ring[PD];
  ScaleRegs6 s6[Q6 ? PD : 1];  // Q6_K: the lane's run scales and d of each slot
  auto load_next = [&](int s) {
    BlockRegs& r = ring[s];
    const int tg = a.t0 + ltl;
    if (Q6) {
      load_rec6(r, s6[Q6 ? s : 0], A.w + ((size_t)tg * A.KB + a.kb0 + lb) * Q6W_REC, lane);
    } else if (FMT == GEMM_TILES) {
      load_rec(r, A.w + ((size_t)tg * A.KB + a.kb0 + lb) * TILE_REC, lane);
    } else {
      const int col = min(16 * tg + c, A.N - 1);
      load_block(r, A.w + ((size_t)col * A.KB + a.kb0 + lb) * BLOCK_BYTES, g);
    }
    if (lu + 1 < ub) {
      ++lu;
      if (++lb == a.nkb) {
        lb = 0;
        ++ltl;
      }
    }
  };
  // the first weight records are in flight while the activations are staged
#pragma unroll
  for (int s = 0; s < PD; ++s)
    if (s < ub - ua) load_next(s);
  if (a.U > 0) stage_x(A.x, A.K, A.M, a.kb0, a.nkb, x_lds, A.x_stride, tid, GEMM_THREADS);
  __syncthreads();
  if (!Q6) {  // the Q4_K min term's sub-block sums (Q6_K has none)
    if (a.U > 0)
      stage_xsum(A.M, a.nkb, xsum_row_bytes(a.nkb), x_lds, A.x_stride, xs_lds, tid, GEMM_THREADS);
    __syncthreads();
  }

  // this wave's parts of the tiles it shares (slot 0, slot 1), held until the
  // stream ends
  floatx4 part0[MT], part1[MT];
  bool has0 = false, has1 = false;
  if (ua < ub) {

    floatx4 acc[MT];
#pragma unroll
    for (int rt = 0; rt < MT; ++rt) acc[rt] = floatx4{0.f, 0.f, 0.f, 0.f};
    int ctl = ua / a.nkb, cb = ua - ctl * a.nkb, cu = ua;
    auto flush = [&]() {
      // the tile is this wave's alone when all its units lie in [ua, ub)
      if (ctl * a.nkb >= ua && (ctl + 1) * a.nkb <= ub) {
#pragma unroll
        for (int rt = 0; rt < MT; ++rt) put(a.t0 + ctl, lane, acc[rt], rt);
      } else if (ctl * a.nkb < ua) {
#pragma unroll
        for (int rt = 0; rt < MT; ++rt) part0[rt] = acc[rt];
        has0 = true;
      } else {
#pragma unroll
        for (int rt = 0; rt < MT; ++rt) part1[rt] = acc[rt];
        has1 = true;
      }
#pragma unroll
      for (int rt = 0; rt < MT; ++rt) acc[rt] = floatx4{0.f, 0.f, 0.f, 0.f};
    };
    auto consume = [&](int s) {
      const char* xab[MT];
      const char* xsb[MT];
#pragma unroll
      for (int rt = 0; rt < MT; ++rt) {
        xab[rt] = xa[rt] + cb * X_BYTES_PER_BLOCK;
        xsb[rt] = xs[rt] + cb * XSUM_BYTES_PER_BLOCK;
      }
      if constexpr (Q6)
        mma_unit6_mt<MT>(ring[s], s6[s], xab, acc);
      else
        mma_unit_mt<MT>(ring[s], g, xab, xsb, k, acc);
      ++cu;
      if (++cb == a.nkb || cu == ub) {
        flush();
        if (cb == a.nkb) {
          cb = 0;
          ++ctl;
        }
      }
    };
    // unit r sits in ring slot r % PD; once consumed, its slot takes unit
    // r + PD, if the wave has one
    const int U = ub - ua;
    for (int r0 = 0; r0 < U; r0 += PD) {
#pragma unroll
      for (int s = 0; s < PD; ++s) {
        if (r0 + s >= U) break;
        consume(s);
        if (r0 + s + PD < U) load_next(s);
      }
    }
  }
  __syncthreads();  // every wave is done with the staged activations
  if (has0) {
#pragma unroll
    for (int rt = 0; rt < MT; ++rt)
      *reinterpret_cast<floatx4*>(slot(wave, 0, rt) + lane * 16) = part0[rt];
  }
  if (has1) {
#pragma unroll
    for (int rt = 0; rt < MT; ++rt)
      *reinterpret_cast<floatx4*>(slot(wave, 1, rt) + lane * 16) = part1[rt];
  }
  __syncthreads();

  // Tiles shared by waves: each holds the start of some wave's range other
  // than at its first unit; taken once, at the first such boundary. The
  // tile's first wave left its part in slot 1, every later wave in slot 0.
  for (int e = tid; e < (SPLIT_WAVES - 1) * MT * 64; e += GEMM_THREADS) {
    const int vb = 1 + (e >> 6) / MT, rt = (e >> 6) % MT, ln = e & 63;
    const int u = wave_begin(a, vb);
    if (u >= a.U || u % a.nkb == 0) continue;
    const int tl = u / a.nkb;
    const int up = wave_begin(a, vb - 1);
    if (vb > 1 && up % a.nkb != 0 && up / a.nkb == tl) continue;
    const int w0 = wave_of_unit(a, tl * a.nkb);
    const int w1 = wave_of_unit(a, (tl + 1) * a.nkb - 1);
    floatx4 v = *reinterpret_cast<const floatx4*>(slot(w0, 1, rt) + ln * 16);
    for (int vv = w0 + 1; vv <= w1; ++vv) {
      if (wave_begin(a, vv) == wave_begin(a, vv + 1)) continue;  // empty range: wrote nothing
      v += *reinterpret_cast<const floatx4*>(slot(vv, 0, rt) + ln * 16);
    }
    put(a.t0 + tl, ln, v, rt);
  }
}

// The second kernel of a K-split call: one wave per (column tile, row tile)
// adds the tile's sk slice partials in slice order and writes Y. It runs
// after the streaming kernel on the same stream, so every partial is in
// memory; no counters are needed.
constexpr int REDUCE_THREADS = 256;
__global__ void __launch_bounds__(REDUCE_THREADS)
    q4k_gemm_reduce(const char* __restrict__ part, float* __restrict__ y, int M, int N, int nt,
                    int sk, int mt) {
  const int task = blockIdx.x * (REDUCE_THREADS / 64) + (threadIdx.x >> 6);
  if (task >= nt * mt) return;
  const int tg = task / mt, rt = task - tg * mt, ln = threadIdx.x & 63;
  const char* base = part + ((size_t)tg * sk * mt + rt) * 1024 + ln * 16;
  const size_t stride = (size_t)mt * 1024;
  floatx4 acc = {0.f, 0.f, 0.f, 0.f};
  constexpr int SB = 8;  // pieces loaded before any is added
  for (int s0 = 0; s0 < sk; s0 += SB) {
    floatx4 v[SB];
#pragma unroll
    for (int i = 0; i < SB; ++i)
      v[i] = *reinterpret_cast<const floatx4*>(base + (size_t)min(s0 + i, sk - 1) * stride);
#pragma unroll
    for (int i = 0; i < SB; ++i)
      if (s0 + i < sk) acc += v[i];
  }
  const int col = 16 * tg + (ln & 15);
  if (col < N) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = 16 * rt + 4 * (ln >> 4) + r;
      if (m < M) y[(size_t)m * N + col] = acc[r];
    }
  }
}

namespace {

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// The second launch (the slice reduction), priced in bytes through one
// compute unit's load path: a launch costs a few microseconds of host and
// queue time, about what 128 KiB take on that path.
constexpr double kLaunchBytes = 131072.0;

GemmPlan make_plan(int M, int N, int K, int G, int fmt) {
  const double rec = fmt == GEMM_Q6W ? (double)Q6W_REC : (double)TILE_REC;
  GemmPlan p;
  p.mt = (M + 15) / 16;
  p.KB = K / QK;
  p.nt = (N + 15) / 16;
  p.G = G < p.nt * p.KB ? G : p.nt * p.KB;  // no more workgroups than units
  G = p.G;
  const size_t contrib = (size_t)SPLIT_WAVES * 2 * p.mt * 1024;
  // Among the splits that fit in LDS, take the one that moves the fewest
  // bytes through the busiest workgroup (a compute unit's load path is the
  // bottleneck): its weight records, its staged activations and the slice
  // partials it stores; with K slices, also one compute unit's share of the
  // partials the reduction reads, 12 KiB for each of its rounds of eight
  // loads (a round trip takes about as long as 12 KiB on that path) and
  // kLaunchBytes for the second launch. nkb = 1 is taken when nothing else
  // fits.
  //
  // The split is chosen for the largest row count a call takes (MK_Q4K_MAX_M),
  // whatever M is: the K slices, and so the order in which every output is
  // summed, depend on N, K and the device only. A row's result is then the
  // same, bit for bit, whether it is multiplied alone or stacked with others.
  const int Mp = MK_Q4K_MAX_M, mtp = (Mp + 15) / 16;
  const size_t contrib_p = (size_t)SPLIT_WAVES * 2 * mtp * 1024;
  auto x_bytes = [](int rows, int nkb) {
    const size_t b = (size_t)rows * (nkb * X_BYTES_PER_BLOCK + X_ROW_PAD) +
                     (size_t)rows * xsum_row_bytes(nkb);
    return (b + 15) & ~(size_t)15;
  };
  double best = -1.0;
  int prev_nkb = -1;
  for (int sk = 1; sk <= p.KB; ++sk) {
    const int nkb = (p.KB + sk - 1) / sk;
    if (nkb == prev_nkb) continue;
    prev_nkb = nkb;
    const int skr = (p.KB + nkb - 1) / nkb;
    const size_t c0 = x_bytes(Mp, nkb);
    int tw_max = 1, umax = 0;
    for (int w = 0; w < G; ++w) {
      const Assign a = assign_split(p.nt, skr, nkb, p.KB, w, G);
      if (a.tw > tw_max) tw_max = a.tw;
      if (a.U > umax) umax = a.U;
    }
    // the contribution slots reuse the activation region after the stream
    const size_t c1 = c0 > contrib_p ? c0 : contrib_p;
    const bool fits = c1 + 256 <= kGemmLdsLimit;
    const double part = (double)mtp * 1024;
    const double bytes = (double)umax * rec + (double)Mp * nkb * X_BYTES_PER_BLOCK +
                         (skr > 1 ? tw_max * part + (double)p.nt * skr * part / G +
                                        (skr + 7) / 8 * 12288.0 + kLaunchBytes
                                  : 0.0);
    if ((fits && (best < 0 || bytes < best)) || (nkb == 1 && best < 0)) {
      best = bytes;
      p.sk = skr;
      p.nkb = nkb;
      p.x_stride = nkb * X_BYTES_PER_BLOCK + X_ROW_PAD;
      p.ok = fits;
    }
  }
  // LDS for the actual rows: their slice of activations, or the slots
  {
    const size_t c0 = x_bytes(M, p.nkb);
    p.lds = c0 > contrib ? c0 : contrib;
  }
  // workspace: the slice partials (no initial contents needed)
  p.part_bytes = p.sk > 1 ? (size_t)p.nt * p.sk * p.mt * 1024 : 0;
  p.part_off = 0;
  p.ws_bytes = p.part_bytes;
  if (p.part_bytes >= (1ull << 32)) p.ok = false;
  return p;
}

std::mutex g_plan_mu;
std::map<std::tuple<int, int, int, int, bool>, GemmPlan> g_plans;

// Dynamic LDS each kernel instantiation has been allowed on each device
// (the attribute is raised only when a plan needs more).
std::mutex g_attr_mu;
std::map<std::pair<const void*, int>, size_t> g_attr_lds;

hipError_t allow_lds(const void* kern, size_t lds) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lk(g_attr_mu);
  size_t& have = g_attr_lds[std::make_pair(kern, dev)];
  if (have >= lds) return hipSuccess;
  e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e == hipSuccess) have = lds;
  return e;
}

template <int MT, int FMT>
hipError_t launch(const GemmPlan& p, const GemmArgs& A, hipStream_t st) {
  auto kern = q4k_gemm_kernel<MT, FMT>;
  hipError_t e = allow_lds((const void*)kern, p.lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(p.G), dim3(GEMM_THREADS), p.lds, st, A);
  e = hipGetLastError();
  if (e != hipSuccess || p.sk == 1) return e;
  const int waves = p.nt * MT;
  hipLaunchKernelGGL(q4k_gemm_reduce, dim3((waves + REDUCE_THREADS / 64 - 1) / (REDUCE_THREADS / 64)),
                     dim3(REDUCE_THREADS), 0, st, A.part, A.y, A.M, A.N, p.nt, p.sk, MT);
  return hipGetLastError();
}

template <int FMT>
hipError_t launch_mt(const GemmPlan& p, const GemmArgs& A, hipStream_t st) {
  switch (p.mt) {
    case 1: return launch<1, FMT>(p, A, st);
    case 2: return launch<2, FMT>(p, A, st);
    case 3: return launch<3, FMT>(p, A, st);
    default: return launch<4, FMT>(p, A, st);
  }
}

}  // namespace

GemmPlan gemm_plan(int M, int N, int K, int G, int fmt) {
  std::lock_guard<std::mutex> lk(g_plan_mu);
  // the row and tile forms cost the same bytes: one plan
  const auto key = std::make_tuple(M, N, K, G, fmt == GEMM_Q6W);
  auto it = g_plans.find(key);
  if (it != g_plans.end()) return it->second;
  const GemmPlan p = make_plan(M, N, K, G, fmt);
  if (g_plans.size() > 4096) g_plans.clear();
  g_plans.emplace(key, p);
  return p;
}

hipError_t gemm_launch(const GemmPlan& p, int fmt, const void* W, const uint16_t* X, float* Y,
                       int M, int N, int K, void* ws, hipStream_t st) {
  GemmArgs A;
  A.w = static_cast<const uint8_t*>(W);
  A.x = X;
  A.y = Y;
  A.part = static_cast<char*>(ws) + p.part_off;
  A.part_bytes = (unsigned)p.part_bytes;
  A.M = M;
  A.N = N;
  A.K = K;
  A.KB = p.KB;
  A.nt = p.nt;
  A.sk = p.sk;
  A.nkb = p.nkb;
  A.G = p.G;
  A.x_stride = p.x_stride;
  switch (fmt) {
    case GEMM_TILES: return launch_mt<GEMM_TILES>(p, A, st);
    case GEMM_Q6W: return launch_mt<GEMM_Q6W>(p, A, st);
    default: return launch_mt<GEMM_ROWS>(p, A, st);
  }
}

}  // namespace mk
