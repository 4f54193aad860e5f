// q4k_step.hip - the decode step as one persistent kernel.
//
// One launch walks every layer's seven Q4_K matrices (the OpenJet post, "RTX
// 3090 one card, four coding agents", paragraph on how parallel decoding
// works: the whole step is one persistent kernel with no per-layer launches,
// and every weight read once multiplies all stacked rows). Per layer there are
// four dependent phases:
//   A: x_l -> q, k, v     B: c(q) -> o     C: c(o) -> gate, up
//   D: c(gate * up) -> down,     x_{l+1} = c(down)
// with c the binary16 round-to-nearest-even cast. Every matrix multiplies the
// row-standardized form of its binary16 input, applied exactly after the
// product: y = (sum x*w - mean * colsum) / sqrt(var + 1e-6).
//
// Work split (G workgroups of 8 waves, one per CU):
//   A phase's columns form 16-wide tiles (gate and up tiles travel as a pair
//   that shares the activation operands). K is cut into sk slices; workgroup
//   w takes slice w % sk and a contiguous run of tiles. It stages the binary16
//   activations of its slice in LDS once (and adds the input's row statistics
//   while doing so); its waves split the run's (tile, super-block) units into
//   equal contiguous ranges and stream them from the tile-record weights
//   through a register ring. Every tile's wave parts stay in LDS until the
//   stream ends and are added in wave order.
//   Slice partials go to the workspace, each word tagged with the layer's
//   parity. Tile t is finished by the workgroup of slice t % sk: it waits
//   until every slice's piece shows the right parity, adds the pieces in
//   slice order, applies the standardization, writes the outputs and the
//   binary16 input of the next phase, adds the tile's row statistics of that
//   input (64-bit fixed-point atomics, order independent) and counts the tile
//   as finished. The next phase starts when every tile of this one is counted
//   finished; its first weight records are in flight by then.
//
// Cross-workgroup memory protocol (no cache flushes or invalidates): data
// another workgroup reads is written with device-coherent stores (sc1) and
// the writer waits for them (s_waitcnt vmcnt(0)) before it adds to a counter;
// readers poll counters with device-coherent loads and read shared data
// either with device-coherent loads (partials, statistics) or, for the phase
// input copies, with ordinary loads of addresses no workgroup touched before
// they were written (one fresh, 256-byte aligned buffer per layer and phase),
// so no cache can hold a stale line of them.
#include <math.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <vector>

#include "mk_q4k.h"
#include "q4k_device.h"
#include "q4k_host.h"
#include "q4k_step.h"

namespace mk {

namespace {

constexpr unsigned long long kTimeoutTicks = 500000000ull;  // 5 s at 100 MHz
constexpr int kStageRound = 10;  // staging chunks a thread loads before using them
// statistics slot values (STAT_SLOTS x M x 2) each thread reads when staging
constexpr int kStatPer = (STAT_SLOTS * STEP_MAX_M * 2 + STEP_THREADS - 1) / STEP_THREADS;

// A statistics word: 32 S + 1 for a share S, its share count, its sum.
__device__ __forceinline__ long long stat_share(unsigned long long s) {
  return (long long)((s << STAT_CNT_BITS) + 1u);
}
__device__ __forceinline__ int stat_count(long long v) {
  return (int)(v & ((1 << STAT_CNT_BITS) - 1));
}
__device__ __forceinline__ unsigned long long stat_sum(long long v) {
  return (unsigned long long)(v >> STAT_CNT_BITS);  // arithmetic: exact for negative sums
}

__device__ __forceinline__ void wait_vm0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Timeline stamp (MK_STEP_TIMELINE builds only): thread 0 stores the wall
// clock for (layer, phase, workgroup, event).
__device__ __forceinline__ void tl_stamp(const StepParams& P, int l, int p, int ev) {
  if constexpr (MK_STEP_TIMELINE) {
    if (threadIdx.x == 0) {
      unsigned long long* tl = reinterpret_cast<unsigned long long*>(P.ws + P.tl_off);
      tl[(((size_t)l * 4 + p) * P.G + blockIdx.x) * TL_EVENTS + ev] = wall_clock64();
    }
  }
}

// Device-coherent (agent-scope) loads of values other workgroups write.
// The pointers are taken as global-address-space ones: through a generic
// pointer the access would be a flat one, which also counts against the LDS
// wait counter and so makes unrelated LDS accesses wait for memory.
template <class T>
__device__ __forceinline__ T ld_dev(const T* p) {
  return __hip_atomic_load((gptr<T>)(const_cast<T*>(p)), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

static_assert(STEP_WAVES == SPLIT_WAVES, "the step splits units like the other streaming kernels");
static_assert(STEP_PD % 2 == 0, "gate and up records take ring slots in pairs");

// The value of another lane of the same 16-lane row (DPP control CTRL: a
// quad permutation, or a rotation of the row).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL,
                                                            0xF, 0xF, false));
}
constexpr int kQuadSwap1 = 0xB1;  // quad lanes 1,0,3,2
constexpr int kQuadSwap2 = 0x4E;  // quad lanes 2,3,0,1
constexpr int kRowRor4 = 0x124;
constexpr int kRowRor8 = 0x128;

// Sum over the 16 lanes of a row, the same in every lane of it (each step
// adds the same two operands in every lane, in either order).
__device__ __forceinline__ float row_sum16(float v) {
  v += dpp_mov<kRowRor8>(v);
  v += dpp_mov<kRowRor4>(v);
  v += dpp_mov<kQuadSwap2>(v);
  v += dpp_mov<kQuadSwap1>(v);
  return v;
}

// Slice-partial words tagged with a layer parity (see PART_FILL).
__device__ __forceinline__ floatx4 tag_parity(const floatx4& v, unsigned par) {
  const u32x4 b = __builtin_bit_cast(u32x4, v);
  return __builtin_bit_cast(floatx4, u32x4{(b.x & ~1u) | par, (b.y & ~1u) | par,
                                           (b.z & ~1u) | par, (b.w & ~1u) | par});
}
__device__ __forceinline__ floatx4 untag(const floatx4& v) {
  const u32x4 b = __builtin_bit_cast(u32x4, v);
  return __builtin_bit_cast(floatx4, u32x4{b.x & ~1u, b.y & ~1u, b.z & ~1u, b.w & ~1u});
}
__device__ __forceinline__ bool arrived(const floatx4& v, unsigned par) {
  const u32x4 b = __builtin_bit_cast(u32x4, v);
  return ((b.x & 1u) == par) && ((b.y & 1u) == par) && ((b.z & 1u) == par) &&
         ((b.w & 1u) == par);
}

__device__ __forceinline__ void set_status(const StepParams& P, int code) {
  int* status = reinterpret_cast<int*>(P.ws + P.status_off);
  int expect = 0;
  __hip_atomic_compare_exchange_strong(status, &expect, code, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
}

// A work split held in LDS, read into wave-uniform registers.
__device__ __forceinline__ Assign lds_assign(const Assign& x) {
  Assign a;
  a.s = uni(x.s);
  a.t0 = uni(x.t0);
  a.tw = uni(x.tw);
  a.kb0 = uni(x.kb0);
  a.nkb = uni(x.nkb);
  a.j = uni(x.j);
  a.gs = uni(x.gs);
  a.U = uni(x.U);
  return a;
}


__device__ __forceinline__ int seg_of(const DevPhase& ph, int tg) {
  return (tg >= uni(ph.seg_t0[1])) + (tg >= uni(ph.seg_t0[2]));
}

// Walks one wave's weight records of a phase: units ua..ub-1 of the
// workgroup (unit u = tile u / nkb, super-block u % nkb), nm records per unit.
// Past the end it keeps pointing at the last record (re-read, never used).
// Moving to the next tile of the same matrix adds a stride; only crossing
// into the next column segment (phase A: q -> k -> v) looks the pointers up.
struct Iter {
  int u, ub, b, q;
  int tg;       // tile (phase numbering)
  int seg_end;  // first tile of the next segment
  unsigned stride;  // bytes from one tile's records to the next
  unsigned rec;     // bytes of one record of the current segment (Q6 walks)
  const uint8_t* base[2];  // record (tg, super-block a.kb0) of each matrix
};

// One layer's entry of the layer table (an LDS copy): its 7 weight pointers
// and which of them are Q6_K.
typedef const DevLayer* WPtrs;

// Record bytes of matrix mi of layer L: Q4_K tile records, or (in a walk
// built for Q6_K, Q6) the Q6_K walk records.
template <bool Q6>
__device__ __forceinline__ unsigned rec_bytes(WPtrs L, int mi) {
  if constexpr (Q6) return (uni((int)L->q6) >> mi) & 1 ? (unsigned)Q6W_REC : (unsigned)TILE_REC;
  return TILE_REC;
}

template <bool Q6>
__device__ __forceinline__ void iter_tile(Iter& it, const DevPhase& ph, WPtrs L,
                                          const Assign& a) {
  const int seg = seg_of(ph, it.tg);
  const int mi = uni(ph.mat0) + seg;
  const unsigned rec = rec_bytes<Q6>(L, mi);
  it.rec = rec;
  it.stride = (unsigned)uni(ph.KB) * rec;
  const size_t off = (size_t)(it.tg - uni(ph.seg_t0[seg])) * it.stride + (size_t)a.kb0 * rec;
  it.seg_end = uni(ph.seg_t0[seg + 1]);
  it.base[0] = uni(L->w[mi]) + off;
  it.base[1] = uni(ph.nm) == 2 ? uni(L->w[mi + 1]) + off : it.base[0];
}

// Start of a wave's walk from st = (first unit, end unit, tile, super-block)
// and sp = (matrix of that tile, record index in it, first tile of the next
// segment), all computed once per launch.
template <bool Q6>
__device__ __forceinline__ void iter_init(Iter& it, const DevPhase& ph, WPtrs L,
                                          const int4& st, const int4& sp) {
  it.u = uni(st.x);
  it.ub = uni(st.y);
  it.q = 0;
  it.tg = uni(st.z);
  it.b = uni(st.w);
  const int mi = uni(sp.x);
  const unsigned rec = rec_bytes<Q6>(L, mi);
  it.rec = rec;
  it.stride = (unsigned)uni(ph.KB) * rec;
  it.seg_end = uni(sp.z);
  const unsigned off = (unsigned)uni(sp.y) * rec;
  it.base[0] = uni(L->w[mi]) + off;
  it.base[1] = uni(ph.nm) == 2 ? uni(L->w[mi + 1]) + off : it.base[0];
}

template <bool Q6>
__device__ __forceinline__ const uint8_t* iter_addr(const Iter& it) {
  return (it.q ? it.base[1] : it.base[0]) + (unsigned)it.b * (Q6 ? it.rec : (unsigned)TILE_REC);
}

template <bool Q6>
__device__ __forceinline__ void iter_next(Iter& it, const DevPhase& ph, WPtrs L,
                                          const Assign& a) {
  const int nm = uni(ph.nm);
  if (++it.q < nm) return;
  if (it.u + 1 >= it.ub) {  // stay on the last record
    it.q = nm - 1;
    return;
  }
  it.q = 0;
  ++it.u;
  if (++it.b < a.nkb) return;
  it.b = 0;
  if (++it.tg < it.seg_end) {
    it.base[0] += it.stride;
    it.base[1] += it.stride;
  } else {
    iter_tile<Q6>(it, ph, L, a);
  }
}

// First unit (of the workgroup's split a) in a Q6_K matrix of layer L in
// phase ph, or a.U when none: Q6_K is allowed only for v (the last segment of
// phase A) and down (phase D), so such units are always the split's tail.
template <bool Q6>
__device__ __forceinline__ int q6_first_unit(const DevPhase& ph, WPtrs L, const Assign& a) {
  if constexpr (!Q6) return a.U;
  const int q6 = uni((int)L->q6);
  const int m0 = uni(ph.mat0), ns = uni(ph.nseg);
  for (int s = 0; s < ns; ++s) {
    if ((q6 >> (m0 + s)) & 1) {
      const int u = (uni(ph.seg_t0[s]) - a.t0) * a.nkb;
      return u < 0 ? 0 : (u > a.U ? a.U : u);
    }
  }
  return a.U;
}

// Issue a phase's first STEP_PD weight records of the wave (fewer if the
// wave has fewer) into ring slots 0.., before the phase's input is ready.
template <bool Q6>
__device__ __forceinline__ void ring_fill(BlockRegs (&ring)[STEP_PD], Iter& it,
                                          const DevPhase& ph, WPtrs L, const Assign& a,
                                          int lane) {
  // Q4_K records only: a wave's Q6_K tail fills its own ring when it gets there
  const int u6 = q6_first_unit<Q6>(ph, L, a);
  const int nrec = ((it.ub < u6 ? it.ub : u6) - it.u) * uni(ph.nm);
#pragma unroll
  for (int s = 0; s < STEP_PD; ++s) {
    if (s < nrec) {
      load_rec(ring[s], iter_addr<Q6>(it), lane);
      iter_next<Q6>(it, ph, L, a);
    }
  }
}

// A wave's record table of one phase, one entry per lane (so the walk needs
// no record iterator and its loop no branches). Lane r holds the address of
// the wave's record r (records past the wave's last repeat it and are never
// read) and the facts of its unit r: the super-block within the slice, whether
// the unit starts a tile, and the byte offset of that tile's contribution
// slot. The walk reads entries with a wave-uniform index (v_readlane). Every
// unit stores its tile's running sum to the slot, so the tile's last unit
// leaves the final one there, and a unit that starts a tile starts from zero.
struct RecTab {
  uint32_t lo, hi;  // record address
  uint32_t info;    // super-block (bits 0-3) | starts a tile (bit 4) | slot offset (bits 8-31)
};
constexpr int TAB_MAX = 64;  // records (and units) of one wave a table holds

template <bool Q6>
__device__ __forceinline__ RecTab build_tab(const DevPhase& ph, WPtrs L, const Assign& a,
                                            int wave, int lane) {
  const int nm = uni(ph.nm);
  const int ua = wave_begin(a, wave), ub = wave_begin(a, wave + 1);
  const int nrec = (ub - ua) * nm;
  const int nkb = a.nkb > 0 ? a.nkb : 1;
  RecTab t;
  {
    const int r = lane < nrec ? lane : (nrec > 0 ? nrec - 1 : 0);
    const int u = ua + (nm == 2 ? r >> 1 : r);
    const int q = nm == 2 ? (r & 1) : 0;
    const int tl = u / nkb;
    const int b = u - tl * nkb;
    const int tg = a.t0 + tl;
    const int seg = (tg >= ph.seg_t0[1]) + (tg >= ph.seg_t0[2]);
    const int mi = ph.mat0 + seg + q;
    const unsigned rec = Q6 && ((L->q6 >> mi) & 1u) ? (unsigned)Q6W_REC : (unsigned)TILE_REC;
    const unsigned idx = (unsigned)(tg - ph.seg_t0[seg]) * (unsigned)ph.KB + (unsigned)(a.kb0 + b);
    const unsigned long long p =
        reinterpret_cast<unsigned long long>(L->w[mi]) + (unsigned long long)idx * rec;
    t.lo = (uint32_t)p;
    t.hi = (uint32_t)(p >> 32);
  }
  {
    const int nu = ub - ua;
    const int u = ua + (lane < nu ? lane : (nu > 0 ? nu - 1 : 0));
    const int tl = u / nkb;
    const int b = u - tl * nkb;
    const unsigned start = (b == 0 || u == ua) ? 1u : 0u;
    const int first = wave_of_unit(a, tl * nkb);
    const unsigned slot = (unsigned)((tl * ph.cmax + (wave - first)) * nm) * 1024u;
    t.info = (unsigned)b | (start << 4) | (slot << 8);
  }
  return t;
}

// (readlane returns an int: each half goes through uint32_t, so that a low
// word with bit 31 set is not sign-extended into the high one)
__device__ __forceinline__ const uint8_t* tab_addr(const RecTab& t, int r) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)t.lo, r);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)t.hi, r);
  return reinterpret_cast<const uint8_t*>(((unsigned long long)hi << 32) | lo);
}

// The table form of ring_fill.
template <bool Q6>
__device__ __forceinline__ void ring_fill_tab(BlockRegs (&ring)[STEP_PD], const RecTab& t,
                                              const DevPhase& ph, WPtrs L, const Assign& a,
                                              int wave, int lane) {
  const int ua = wave_begin(a, wave), ub = wave_begin(a, wave + 1);
  const int u6 = q6_first_unit<Q6>(ph, L, a);
  const int nrec = ((ub < u6 ? ub : u6) - ua) * uni(ph.nm);
#pragma unroll
  for (int s = 0; s < STEP_PD; ++s)
    if (s < nrec) load_rec(ring[s], tab_addr(t, s), lane);
}

// The table form of phase_compute (the same products, sums and contribution
// slots; the waves' parts of a tile are added in wave order afterwards).
template <int NM, bool Q6>
__device__ __forceinline__ void phase_compute_tab(BlockRegs (&ring)[STEP_PD], const RecTab& t,
                                                  const DevPhase& ph, WPtrs L,
                                                  const Assign& a, int wave, int lane,
                                                  const char* xa_lane, const char* xs_lane,
                                                  char* contrib, const UnpackConsts& k) {
  const int g = lane >> 4;
  const int ua = wave_begin(a, wave), ub = wave_begin(a, wave + 1);
  const int u6 = q6_first_unit<Q6>(ph, L, a);
  const int u4 = ub < u6 ? ub : (ua > u6 ? ua : u6);
  const int U = (u4 - ua) * NM;  // Q4_K records
  if (U <= 0 && (!Q6 || u4 >= ub)) return;
  floatx4 acc[NM];
#pragma unroll
  for (int q = 0; q < NM; ++q) acc[q] = floatx4{0.f, 0.f, 0.f, 0.f};
  char* slot_lane = contrib + lane * 16;
  // unit uu of the wave (uniform): its super-block, a fresh sum at a tile's
  // first unit, the product, and the running sum to the tile's slot
  auto unit_info = [&](int uu, int& cb) {
    const unsigned inf = (uint32_t)__builtin_amdgcn_readlane((int)t.info, uu);
    cb = (int)(inf & 15u);
    const bool fresh = (inf & 16u) != 0;  // a select, not a branch
#pragma unroll
    for (int q = 0; q < NM; ++q)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[q][e] = fresh ? 0.f : acc[q][e];
    return slot_lane + (inf >> 8);
  };
  auto consume = [&](int s, int uu) {
    int cb;
    char* sl = unit_info(uu, cb);
    mma_unit<NM>(&ring[s], g, xa_lane + cb * X_BYTES_PER_BLOCK,
                 xs_lane + cb * XSUM_BYTES_PER_BLOCK, k, acc);
#pragma unroll
    for (int q = 0; q < NM; ++q) *reinterpret_cast<floatx4*>(sl + q * 1024) = acc[q];
  };
  // Record r sits in ring slot r % STEP_PD; once consumed, its slot takes
  // record r + STEP_PD, if the wave has one (no load past the range).
  int r0 = 0;
  for (; r0 + 2 * STEP_PD <= U; r0 += STEP_PD) {
#pragma unroll
    for (int s = 0; s < STEP_PD; s += NM) {
      consume(s, (r0 + s) / NM);
#pragma unroll
      for (int q = 0; q < NM; ++q) load_rec(ring[s + q], tab_addr(t, r0 + s + q + STEP_PD), lane);
    }
  }
  for (; r0 < U; r0 += STEP_PD) {
#pragma unroll
    for (int s = 0; s < STEP_PD; s += NM) {
      if (r0 + s >= U) break;
      consume(s, (r0 + s) / NM);
      if (r0 + s + STEP_PD < U) {
#pragma unroll
        for (int q = 0; q < NM; ++q)
          load_rec(ring[s + q], tab_addr(t, r0 + s + q + STEP_PD), lane);
      }
    }
  }
  if constexpr (Q6) {
    // the Q6_K tail (one record per unit), records U.. of the table, through
    // the same ring slots (the Q4_K records are all used)
    if constexpr (NM == 1) {
      const int U6 = ub - u4;
      if (U6 > 0) {
        ScaleRegs6 s6[STEP_PD];
#pragma unroll
        for (int s = 0; s < STEP_PD; ++s)
          if (s < U6) load_rec6(ring[s], s6[s], tab_addr(t, U + s), lane);
        auto consume6 = [&](int s, int uu) {
          int cb;
          char* sl = unit_info(uu, cb);
          mma_unit6(ring[s], s6[s], xa_lane + cb * X_BYTES_PER_BLOCK, acc[0]);
          *reinterpret_cast<floatx4*>(sl) = acc[0];
        };
        int q0 = 0;
        for (; q0 + 2 * STEP_PD <= U6; q0 += STEP_PD) {
#pragma unroll
          for (int s = 0; s < STEP_PD; ++s) {
            consume6(s, U + q0 + s);
            load_rec6(ring[s], s6[s], tab_addr(t, U + q0 + s + STEP_PD), lane);
          }
        }
        for (; q0 < U6; q0 += STEP_PD) {
#pragma unroll
          for (int s = 0; s < STEP_PD; ++s) {
            if (q0 + s >= U6) break;
            consume6(s, U + q0 + s);
            if (q0 + s + STEP_PD < U6)
              load_rec6(ring[s], s6[s], tab_addr(t, U + q0 + s + STEP_PD), lane);
          }
        }
      }
    }
  }
}

// Stream the wave's units and multiply them against the staged activations.
// A tile the wave computes alone goes straight to its slice partial block in
// the workspace (one 16-byte store per lane, issued while the stream goes
// on); a tile shared with other waves leaves its part in the LDS contribution
// slot (tile, wave - first wave of the tile). Per lane one floatx4: rows
// 4*(lane/16)+r, column lane%16.
template <int NM, bool Q6>
__device__ __forceinline__ void phase_compute(BlockRegs (&ring)[STEP_PD], Iter& it,
                                              const DevPhase& ph, WPtrs L,
                                              const Assign& a, int wave, int lane,
                                              const char* xa_lane, const char* xs_lane,
                                              char* contrib, const UnpackConsts& k) {
  const int g = lane >> 4;
  const int ua = wave_begin(a, wave), ub = wave_begin(a, wave + 1);
  // units [ua, u4) are Q4_K, [u4, ub) Q6_K (a Q6_K matrix is always the
  // phase's tail, and its phase has one record per unit)
  const int u6 = q6_first_unit<Q6>(ph, L, a);
  const int u4 = ub < u6 ? ub : (ua > u6 ? ua : u6);
  const int U = (u4 - ua) * NM;  // Q4_K records
  if (U <= 0 && (!Q6 || u4 >= ub)) return;
  floatx4 acc[NM];
#pragma unroll
  for (int q = 0; q < NM; ++q) acc[q] = floatx4{0.f, 0.f, 0.f, 0.f};
  int ctl = ua / a.nkb;
  int cb = ua - ctl * a.nkb;
  int cu = ua;
  auto flush = [&]() {
    const int first = wave_of_unit(a, ctl * a.nkb);
    char* slot = contrib + ((size_t)(ctl * ph.cmax + (wave - first)) * NM) * 1024 + lane * 16;
#pragma unroll
    for (int q = 0; q < NM; ++q) {
      *reinterpret_cast<floatx4*>(slot + q * 1024) = acc[q];
      acc[q] = floatx4{0.f, 0.f, 0.f, 0.f};
    }
  };
  // after the product of unit cu: the tile's part goes out when the tile or
  // the wave's range ends
  auto advance = [&]() {
    ++cu;
    if (++cb == a.nkb || cu == ub) {
      flush();
      if (cb == a.nkb) {
        cb = 0;
        ++ctl;
      }
    }
  };
  auto consume = [&](int s) {
    mma_unit<NM>(&ring[s], g, xa_lane + cb * X_BYTES_PER_BLOCK, xs_lane + cb * XSUM_BYTES_PER_BLOCK,
                 k, acc);
    advance();
  };
  // Record r sits in ring slot r % STEP_PD; once consumed, its slot takes
  // record r + STEP_PD, if the wave has one (no load past the range). In the
  // steady-state loop every refill exists, so each use waits only for its own
  // slot's loads; the last groups refill conditionally.
  int r0 = 0;
  for (; r0 + 2 * STEP_PD <= U; r0 += STEP_PD) {
#pragma unroll
    for (int s = 0; s < STEP_PD; s += NM) {
      consume(s);
#pragma unroll
      for (int q = 0; q < NM; ++q) {
        load_rec(ring[s + q], iter_addr<Q6>(it), lane);
        iter_next<Q6>(it, ph, L, a);
      }
    }
  }
  for (; r0 < U; r0 += STEP_PD) {
#pragma unroll
    for (int s = 0; s < STEP_PD; s += NM) {
      if (r0 + s >= U) break;
      consume(s);
      if (r0 + s + STEP_PD < U) {
#pragma unroll
        for (int q = 0; q < NM; ++q) {
          load_rec(ring[s + q], iter_addr<Q6>(it), lane);
          iter_next<Q6>(it, ph, L, a);
        }
      }
    }
  }
  if constexpr (Q6) {
    // the Q6_K tail, through the same ring slots (the Q4_K records are all
    // used), refilled here: the iterator stands at the first Q6_K record
    // once the Q4_K records are all loaded
    if constexpr (NM == 1) {
      const int U6 = ub - u4;
      if (U6 > 0) {
        ScaleRegs6 s6[STEP_PD];
#pragma unroll
        for (int s = 0; s < STEP_PD; ++s) {
          if (s < U6) {
            load_rec6(ring[s], s6[s], iter_addr<Q6>(it), lane);
            iter_next<Q6>(it, ph, L, a);
          }
        }
        auto consume6 = [&](int s) {
          mma_unit6(ring[s], s6[s], xa_lane + cb * X_BYTES_PER_BLOCK, acc[0]);
          advance();
        };
        int q0 = 0;
        for (; q0 + 2 * STEP_PD <= U6; q0 += STEP_PD) {
#pragma unroll
          for (int s = 0; s < STEP_PD; ++s) {
            consume6(s);
            load_rec6(ring[s], s6[s], iter_addr<Q6>(it), lane);
            iter_next<Q6>(it, ph, L, a);
          }
        }
        for (; q0 < U6; q0 += STEP_PD) {
#pragma unroll
          for (int s = 0; s < STEP_PD; ++s) {
            if (q0 + s >= U6) break;
            consume6(s);
            if (q0 + s + STEP_PD < U6) {
              load_rec6(ring[s], s6[s], iter_addr<Q6>(it), lane);
              iter_next<Q6>(it, ph, L, a);
            }
          }
        }
      }
    }
  }
}

// Stage the binary16 activations of slice a ([M][K] at src, natural order)
// into LDS in the MFMA order (see q4k_device.h), with the sub-block sums the
// min term multiplies (each as split_xsum's three binary16 parts). Each thread loads
// up to R 8-wide chunks, all in one round; the four chunks of one 32-value
// sub-block sit in four consecutive lanes, which add their fp32 chunk sums
// with two lane exchanges. The row statistics of the whole input (STAT_SLOTS
// slots of [M][2] integer sums at st, complete before the phase starts) are
// loaded in the same round and added into tot_s (cleared by the caller) with
// LDS integer atomics; the finishing of the phase reads the totals.
template <int R>
__device__ __forceinline__ void stage_rounds(const uint16_t* src, int K, int M, const Assign& a,
                                            const long long* st, unsigned long long* tot_s,
                                            char* x_lds, int x_stride, char* xs_lds,
                                            int xs_row, int* cnt_s, int tid) {
  const int cpr = a.nkb * 32;  // 8-wide chunks per row
  const int items = M * cpr;   // at most STEP_THREADS * R
  // row of chunk index x < 2^16: x * magic / 2^32 (cpr < 2^16)
  const unsigned magic = 0xFFFFFFFFu / (unsigned)cpr + 1u;
  // every load is unconditional (indices clamped to the last valid one), so
  // they issue back to back; the statistics first
  const int nv = STAT_SLOTS * M * 2;  // a multiple of 64
  long long pv[kStatPer];
#pragma unroll
  for (int i = 0; i < kStatPer; ++i) pv[i] = ld_dev(st + min(i * STEP_THREADS + tid, nv - 1));
  u32x4 hv[R];
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const int it = min(i * STEP_THREADS + tid, items - 1);
    const int m = __umulhi((unsigned)it, magic);
    const int ch = it - m * cpr;
    const int k = (a.kb0 + (ch >> 5)) * QK + (ch & 31) * 8;
    hv[i] = *to_global(reinterpret_cast<const u32x4*>(src + (size_t)m * K + k));
  }
  const half2v one2 = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
  for (int i = 0; i < R; ++i) {
    if (i * STEP_THREADS + uni(tid & ~63) >= items) continue;
    const int it = i * STEP_THREADS + tid;
    const bool ok = it < items;  // the same for the four lanes of a sub-block
    const int m = __umulhi((unsigned)(ok ? it : items - 1), magic);
    const int ch = (ok ? it : items - 1) - m * cpr;
    const int b = ch >> 5;
    const int kk = (ch & 31) * 8;
    const u32x4 h = hv[i];
    // fp32 sum of the chunk's 8 values (pairwise dot products with 1), then
    // of the sub-block's 4 chunks
    float sum = __builtin_amdgcn_fdot2(bit_cast_<half2v>(h.x), one2, 0.f, false);
    sum = __builtin_amdgcn_fdot2(bit_cast_<half2v>(h.y), one2, sum, false);
    sum = __builtin_amdgcn_fdot2(bit_cast_<half2v>(h.z), one2, sum, false);
    sum = __builtin_amdgcn_fdot2(bit_cast_<half2v>(h.w), one2, sum, false);
    sum += dpp_mov<kQuadSwap1>(sum);
    sum += dpp_mov<kQuadSwap2>(sum);
    if (!ok) continue;
    u32x4 o;  // element order 0,2,1,3,4,6,5,7
    o.x = (h.x & 0xFFFFu) | (h.y << 16);
    o.y = (h.x >> 16) | (h.y & 0xFFFF0000u);
    o.z = (h.z & 0xFFFFu) | (h.w << 16);
    o.w = (h.z >> 16) | (h.w & 0xFFFF0000u);
    const int gq = kk >> 6, hb = (kk >> 5) & 1, u = (kk >> 3) & 3;
    *reinterpret_cast<u32x4*>(x_lds + (size_t)m * x_stride + b * X_BYTES_PER_BLOCK + gq * 128 +
                              (2 * u + hb) * 16) = o;
    if ((ch & 3) == 0)
      put_xsum(xs_lds + (size_t)m * xs_row + b * XSUM_BYTES_PER_BLOCK, kk >> 5, split_xsum(sum));
  }
  int cnt = 0;  // shares counted in this thread's words
#pragma unroll
  for (int i = 0; i < kStatPer; ++i)
    if (i * STEP_THREADS + uni(tid & ~63) < nv) {
      cnt += stat_count(pv[i]);
      atomicAdd(&tot_s[(i * STEP_THREADS + tid) % (2 * M)], stat_sum(pv[i]));
    }
  // the wave's count (exact in fp32) into the workgroup's
  const int rs = (int)row_sum16((float)cnt);
  const int wc = __builtin_amdgcn_readlane(rs, 0) + __builtin_amdgcn_readlane(rs, 16) +
                 __builtin_amdgcn_readlane(rs, 32) + __builtin_amdgcn_readlane(rs, 48);
  if ((tid & 63) == 0) atomicAdd(cnt_s, wc);
}

// Staging with the number of load rounds the slice needs (one per
// STEP_THREADS chunks; the host plan keeps it at most kStageRound), so that
// every issued load is a useful one.
__device__ __forceinline__ void stage_slice(const uint16_t* src, int K, int M, const Assign& a,
                                            const long long* st, unsigned long long* tot_s,
                                            char* x_lds, int x_stride, char* xs_lds,
                                            int xs_row, int* cnt_s, int tid) {
  static_assert(kStageRound == 10, "one instantiation per round count");
  const int r = uni((M * a.nkb * 32 + STEP_THREADS - 1) / STEP_THREADS);
#define MK_STAGE(RR) \
  stage_rounds<RR>(src, K, M, a, st, tot_s, x_lds, x_stride, xs_lds, xs_row, cnt_s, tid)
  if (r > 7) MK_STAGE(10);
  else if (r > 5) MK_STAGE(7);
  else if (r > 4) MK_STAGE(5);
  else if (r > 3) MK_STAGE(4);
  else if (r > 2) MK_STAGE(3);
  else if (r > 1) MK_STAGE(2);
  else MK_STAGE(1);
#undef MK_STAGE
}

// round(v) as a 64-bit integer for |v| < 2^51: adding 1.5 * 2^52 leaves the
// rounded value (ties to even) in the low mantissa bits.
__device__ __forceinline__ long long round_i64(double v) {
  const double t = v + 6755399441055744.0;  // 1.5 * 2^52
  return __builtin_bit_cast(long long, t) - 0x4338000000000000ll;
}

// Mean and 1/sqrt(var + 1e-6) of row m of a phase input from its integer
// statistics totals (sum x * 2^24, sum x^2 * 2^20 over K values): the
// totals and products in double, the reciprocal square root in fp32.
__device__ __forceinline__ float2 row_moments(const unsigned long long* tot_s, int m,
                                              double inv_k) {
  const double mean = (double)(long long)tot_s[2 * m] * (inv_k * (1.0 / STAT_SCALE_SUM));
  const double e2 = (double)(long long)tot_s[2 * m + 1] * (inv_k * (1.0 / STAT_SCALE_SQ));
  const double var = fmax(__builtin_fma(-mean, mean, e2), 0.0);
  return float2{(float)mean, __builtin_amdgcn_rsqf((float)(var + 1e-6))};
}

// Row m's (mean, scale) pair of a phase: the products become
// (z - mean * colsum) * scale (see NORM_STD, NORM_RMS, NORM_NONE).
__device__ __forceinline__ float2 phase_moments(const unsigned long long* tot_s, int m,
                                                const DevPhase& ph) {
  if (ph.norm == NORM_STD) return row_moments(tot_s, m, ph.inv_k);
  if (ph.norm == NORM_NONE) return float2{0.f, 1.f};
  const double ss = (double)(long long)tot_s[2 * m] * 4294967296.0 + (double)(long long)tot_s[2 * m + 1];
  const double ms = ss * (ph.inv_k * (1.0 / RMS_SCALE));
  return float2{0.f, __builtin_amdgcn_rsqf((float)(ms + 1e-6))};
}

// Wait until every tile of the phases up to (l, p) has been counted finished.
__device__ __forceinline__ bool wait_done(const StepParams& P, const DevPhase* PH, int l, int p,
                                          int* abort_s) {
  if (threadIdx.x < 64) {
    const unsigned* done = reinterpret_cast<const unsigned*>(P.ws + P.done_off);
    const int* status = reinterpret_cast<const int*>(P.ws + P.status_off);
    const int c = threadIdx.x;
    unsigned per_layer = 0, upto = 0;
    for (int q = 0; q < 4; ++q) {
      const int nt = PH[q].nt;
      const unsigned nc = (unsigned)(nt / DONE_CTRS + (c < nt % DONE_CTRS ? 1 : 0));
      per_layer += nc;
      if (q <= p) upto += nc;
    }
    const unsigned target = (unsigned)l * per_layer + upto;
    const unsigned long long t0 = wall_clock64();
    int n = 0;
    bool bad = false;
    while (ld_dev(done + (size_t)c * CTR_STRIDE) < target) {
      __builtin_amdgcn_s_sleep(1);
      if ((++n & 63) == 0) {
        if (ld_dev(status) != 0) {
          bad = true;
          break;
        }
        if (wall_clock64() - t0 > kTimeoutTicks) {
          set_status(P, MK_ETIMEOUT);
          bad = true;
          break;
        }
      }
    }
    const bool any_bad = __any(bad);
    if (threadIdx.x == 0) *abort_s = any_bad ? 1 : 0;
  }
  __syncthreads();
  return *abort_s == 0;
}

// Finish the tiles this workgroup is the finisher of: add the sk slice
// partials of each tile in slice order, write the outputs, the consumer copy
// and the row statistics. One task per (tile, lane): the lane's 4 rows of one
// column, loaded as one 16-byte piece per slice and matrix. A thread takes two
// tasks at a time with all their loads in flight together. The statistics of
// each (tile, row) are summed over the tile's 16 columns in fp32 (fixed
// order), rounded to fixed point, added in LDS as integers and sent with one
// atomic per (row, sum).
// Reload a slice partial piece until every one of its words carries this
// layer's parity (each word is written once per layer, so such a piece is
// complete). Gives up when another workgroup has recorded a failure or the
// wall-clock limit passes.
__device__ __forceinline__ floatx4 await_piece(const StepParams& P, __amdgpu_buffer_rsrc_t pr,
                                               unsigned off, floatx4 v, unsigned par,
                                               unsigned long long t0, int* abort_s) {
  int n = 0;
  while (!arrived(v, par)) {
    __builtin_amdgcn_s_sleep(1);
    v = ld4_dev(pr, off);
    if ((++n & 63) == 0) {
      if (ld_dev(reinterpret_cast<const int*>(P.ws + P.status_off)) != 0) {
        *abort_s = 1;
        break;
      }
      if (wall_clock64() - t0 > kTimeoutTicks) {
        set_status(P, MK_ETIMEOUT);
        *abort_s = 1;
        break;
      }
    }
  }
  return v;
}

// Residual-walk operands of one finished tile column, loaded with the
// partial pieces: the four rows of the residual entering the add (hin) and
// the norm weight of the next input at the column (gv).
struct ResCol {
  float hin[4];
  float gv;
};

// One finished tile column (lane ln: column ln % 16, rows 4(ln/16)..+3) of
// the phase: z holds the products with the binary16 input x of the phase.
// The matrix output is the product with the row-normed input,
//   y[m][n] = scale_m * (z[m][n] - mean_m * colsum[n]),
// written to the layer outputs (mean 0 and no column sums outside the
// standardization). For the matrices that feed the next phase, the next
// phase's input is a binary16 cast, written as pairs of columns with
// device-coherent 32-bit stores:
//   MODE 0: of y (of y_gate * y_up, taken in fp32, for the paired phase);
//           the row sums of the cast values go into the statistics;
//   MODE 1 (residual walk), by phase: A: of y (q); B and D: the residual
//           add h_new = h_in + y is written, and the cast is of h_new times
//           the next norm weight, the statistics summing h_new^2; C: of
//           silu(y_gate) * y_up in fp32.
// Statistics go into the workgroup's LDS integer sums (fixed point).
template <int NM, int MODE>
__device__ __forceinline__ void fixup_finish(const StepParams& P, const DevPhase& ph, int p,
                                             const DevLayer* L, uint16_t* xn, bool stats,
                                             float* h_new, const ResCol& rc, int tg, int ln,
                                             const floatx4* z, const float* csum,
                                             const float2* mom_s, unsigned long long* wst) {
  const int M = P.M;
  const int seg = __builtin_amdgcn_readfirstlane(seg_of(ph, tg));  // uniform per wave
  const int nseg = ph.seg_n[seg];
  const int cs = (tg - ph.seg_t0[seg]) * 16 + (ln & 15);
  const int g = ln >> 4;
  const bool feeds = xn != nullptr && seg == 0;  // k and v feed nothing
  const bool res = MODE == 1 && (p == 1 || p == 3);
  float* yp[NM];
#pragma unroll
  for (int q = 0; q < NM; ++q) yp[q] = L->y[ph.mat0 + seg + q];
  const int Kn = ph.seg_n[0];  // width of the next phase's input
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(xn, (unsigned)(M * Kn * 2));
  const __amdgpu_buffer_rsrc_t hr = make_rsrc(h_new, (unsigned)(M * nseg * 4));
  float s1[4], s2[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int m = 4 * g + r;
    const bool valid = m < M && cs < nseg;
    const float2 mv = mom_s[m];  // rows past M hold zeros (never stored)
    const float mu = mv.x, iv = mv.y;
    float y[NM];
#pragma unroll
    for (int q = 0; q < NM; ++q) y[q] = __builtin_fmaf(-mu, csum[q], z[q][r]) * iv;
    if (valid) {
#pragma unroll
      for (int q = 0; q < NM; ++q) to_global(yp[q])[(size_t)m * nseg + cs] = y[q];
    }
    float hv = 0.f, hs = 0.f;
    if (res) {
      // read in a later phase by other workgroups: device-coherent store
      const float hn = rc.hin[r] + y[0];
      if (valid)
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, hn), hr,
                                              (unsigned)((m * nseg + cs) * 4), 0, kCoherent);
      hs = valid ? hn : 0.f;
    }
    if (feeds) {
      // the value cast is the fp32 one (see above): the empty asm keeps the
      // compiler from fusing the last multiply into a mixed-precision op
      // that rounds once, straight to binary16
      float v;
      if (MODE == 1 && res)
        v = (rc.hin[r] + y[0]) * rc.gv;
      else if (MODE == 1 && NM == 2)
        v = y[0] / (1.f + expf(-y[0])) * y[NM - 1];
      else
        v = NM == 2 ? y[0] * y[NM - 1] : y[0];
      asm volatile("" : "+v"(v));
      const _Float16 h = (_Float16)v;
      const int hb = bit_cast_<uint16_t>(h);
      const int hp = __builtin_amdgcn_mov_dpp(hb, kQuadSwap1, 0xF, 0xF, false);  // column cs ^ 1
      if (valid && (cs & 1) == 0)
        __builtin_amdgcn_raw_buffer_store_b32((uint32_t)(hb & 0xFFFF) | ((uint32_t)hp << 16), xr,
                                              (unsigned)((m * Kn + cs) * 2), 0, kCoherent);
      if (MODE == 1 && valid && (hb & 0x7C00) == 0x7C00)
        set_status(P, MK_ERANGE);  // the cast overflowed (or met a NaN)
      hv = valid ? (float)h : 0.f;
    }
    s1[r] = MODE == 0 ? hv : 0.f;
    s2[r] = MODE == 0 ? hv * hv : hs * hs;
  }
  if (!stats) return;
  if (MODE == 0 && !feeds) return;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    if (MODE == 0) s1[r] = row_sum16(s1[r]);
    s2[r] = row_sum16(s2[r]);
  }
  if ((ln & 15) == 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = 4 * g + r;
      if (m >= M) break;
      if (MODE == 0) {
        const double f1 = (double)s1[r] * STAT_SCALE_SUM, f2 = (double)s2[r] * STAT_SCALE_SQ;
        if (!(fabs(f1) < STAT_TERM_MAX) || !(f2 < STAT_TERM_MAX)) {
          set_status(P, MK_ERANGE);  // an overflowed cast or values too large to sum
        } else {
          atomicAdd(&wst[2 * m], (unsigned long long)round_i64(f1));
          atomicAdd(&wst[2 * m + 1], (unsigned long long)round_i64(f2));
        }
      } else {
        const double sq = (double)s2[r];
        if (!(sq < RMS_TERM_MAX)) {
          set_status(P, MK_ERANGE);  // a residual too large to sum (or not finite)
        } else {
          const double t = __builtin_rint(sq * RMS_SCALE);
          const double hi = __builtin_floor(t * (1.0 / 4294967296.0));
          const double lo = __builtin_fma(-hi, 4294967296.0, t);
          atomicAdd(&wst[2 * m], (unsigned long long)(long long)hi);
          atomicAdd(&wst[2 * m + 1], (unsigned long long)(long long)lo);
        }
      }
    }
  }
}

// Column sums of the matrices of tile tg at lane ln's column (they follow
// the tile records; the column is always inside the padded tile range).
template <int NM>
__device__ __forceinline__ void load_colsum(const DevPhase& ph, const DevLayer* L, int tg, int ln,
                                            float* csum) {
  const int seg = __builtin_amdgcn_readfirstlane(seg_of(ph, tg));
  const int cs = (tg - ph.seg_t0[seg]) * 16 + (ln & 15);
  const int mi = ph.mat0 + seg;
  const unsigned off = (uni((int)L->q6) >> mi) & 1 ? ph.cs_off6[seg] : ph.cs_off[seg];
#pragma unroll
  for (int q = 0; q < NM; ++q)
    csum[q] = to_global(reinterpret_cast<const float*>(L->w[mi + q] + off))[cs];
}

// The next phase's input buffer (binary16 [M][Kn]) and the statistics slots
// of it, after phase p of layer l; the last layer's down projection writes
// x_out and no statistics.
template <int MODE>
__device__ __forceinline__ uint16_t* next_input(const StepParams& P, const DevLayer* ltab, int l,
                                                int p) {
  // both candidates are read and the value selected (a selected address
  // would make the compiler read it with a flat load)
  const int ln = l + 1 < P.n_layers ? l + 1 : l;
  uint16_t* nx = uni(p < 3 ? ltab[l].x[p + 1] : ltab[ln].x[0]);
  uint16_t* xo = MODE == 0 ? uni(P.x_out) : nullptr;  // the residual walk ends in h
  return (p == 3 && l + 1 >= P.n_layers) ? xo : nx;
}

template <int NM, int MODE>
__device__ __forceinline__ void fixup_tiles(const StepParams& P, const DevPhase& ph, int p, int l,
                                            const DevLayer* ltab, const Assign& a, int ffirst,
                                            int nfin, unsigned long long* wst,
                                            const float2* mom_s, int* abort_s, int tid) {
  const int M = P.M;
  const DevLayer* L = &ltab[l];
  const __amdgpu_buffer_rsrc_t pr = make_rsrc(P.ws + ph.part_off, ph.part_bytes);
  uint16_t* xn = next_input<MODE>(P, ltab, l, p);
  // MODE 0: every next input but x_out has statistics; MODE 1: the normed
  // ones (after B: gate/up's input; after D: the next layer's q/k/v input)
  const bool stats = MODE == 0 ? (p < 3 || l + 1 < P.n_layers)
                               : (p == 1 || (p == 3 && l + 1 < P.n_layers));
  // residual walk, B and D: the residual entering the add, its output and
  // the next input's norm weight (all [M][H] / [H], read at the tile's columns)
  const bool res = MODE == 1 && (p == 1 || p == 3);
  const float* h_in = nullptr;
  float* h_new = nullptr;
  const float* gn = nullptr;
  if (res) {
    const int lg = l + 1 < P.n_layers ? l + 1 : l;
    h_in = p == 1 ? (l == 0 ? P.h0 : ltab[l > 0 ? l - 1 : 0].h[1]) : L->h[0];
    h_new = p == 1 ? L->h[0] : L->h[1];
    gn = p == 1 ? L->g[1] : ltab[lg].g[0];  // unused after the last layer
    h_in = uni(h_in);
    h_new = uni(h_new);
    gn = uni(gn);
  }
  const int tasks = nfin * 64;
  const unsigned par = (unsigned)l & 1u;
  const unsigned long long t0 = wall_clock64();
  // pieces loaded per round: every load of a round is issued, unconditionally
  // (slices past sk re-read the last one), before any is waited for
  constexpr int PR = 8 / NM;
  for (int t = tid; t < tasks; t += STEP_THREADS) {  // uniform per wave
    const int ln = t & 63;
    const int tg = a.t0 + ffirst + (t >> 6) * ph.sk;
    const unsigned base = (unsigned)tg * ph.sk * NM * 1024u + ln * 16;
    const bool rows_ok = 4 * (ln >> 4) < M;  // lanes holding only rows past M do not wait
    float csum[NM];
    ResCol rc = {};
    if (MODE == 0) {
      load_colsum<NM>(ph, L, tg, ln, csum);
    } else {
#pragma unroll
      for (int q = 0; q < NM; ++q) csum[q] = 0.f;  // no mean term
      if (res) {
        // clamped, so every lane loads (rows past M and columns past N are
        // never stored)
        // h_in was written by other workgroups (device-coherent loads)
        const int cs = min((tg - ph.seg_t0[0]) * 16 + (ln & 15), ph.seg_n[0] - 1);
        const __amdgpu_buffer_rsrc_t hir = make_rsrc(h_in, (unsigned)(M * ph.seg_n[0] * 4));
#pragma unroll
        for (int r = 0; r < 4; ++r)
          rc.hin[r] = __builtin_bit_cast(
              float, __builtin_amdgcn_raw_buffer_load_b32(
                         hir, (unsigned)((min(4 * (ln >> 4) + r, M - 1) * ph.seg_n[0] + cs) * 4), 0,
                         kCoherent));
        rc.gv = to_global(gn)[cs];
      }
    }
    floatx4 y[NM];
#pragma unroll
    for (int q = 0; q < NM; ++q) y[q] = floatx4{0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < ph.sk; s0 += PR) {
      floatx4 v[PR][NM];
#pragma unroll
      for (int i = 0; i < PR; ++i)
#pragma unroll
        for (int q = 0; q < NM; ++q)
          v[i][q] = ld4_dev(pr, base + ((unsigned)min(s0 + i, ph.sk - 1) * NM + q) * 1024u);
      // wait for late slices and add in slice order
#pragma unroll
      for (int i = 0; i < PR; ++i) {
        if (s0 + i >= ph.sk) break;
#pragma unroll
        for (int q = 0; q < NM; ++q) {
          floatx4 u = v[i][q];
          if (rows_ok && !arrived(u, par))
            u = await_piece(P, pr, base + ((s0 + i) * NM + q) * 1024u, u, par, t0, abort_s);
          y[q] += untag(u);
        }
      }
    }
    fixup_finish<NM, MODE>(P, ph, p, L, xn, stats, h_new, rc, tg, ln, y, csum, mom_s, wst);
  }
}

// Wait until every workgroup has added its share of the layer-0 input
// statistics (once per launch, before the first phase's finishing).
__device__ __forceinline__ bool wait_start(const StepParams& P, int* abort_s) {
  if (threadIdx.x == 0) {
    const unsigned* ctr = reinterpret_cast<const unsigned*>(P.ws + P.start_off);
    const int* status = reinterpret_cast<const int*>(P.ws + P.status_off);
    const unsigned long long t0 = wall_clock64();
    int n = 0, bad = 0;
    while (ld_dev(ctr) < (unsigned)P.G) {
      __builtin_amdgcn_s_sleep(1);
      if ((++n & 63) == 0) {
        if (ld_dev(status) != 0) {
          bad = 1;
          break;
        }
        if (wall_clock64() - t0 > kTimeoutTicks) {
          set_status(P, MK_ETIMEOUT);
          bad = 1;
          break;
        }
      }
    }
    *abort_s = bad;
  }
  __syncthreads();
  return *abort_s == 0;
}

// Statistics of the phase input that were not complete when the slice was
// staged: wave 0 reloads every word until all shares are in (every word of
// a slot counts one share per workgroup of the slot, 2 M G in all) and adds
// them up again into tot_s. Returns false if the walk is aborted.
__device__ __forceinline__ bool reload_stats(const StepParams& P, const long long* st,
                                             unsigned long long* tot_s, int lane) {
  const int M = P.M, nv = STAT_SLOTS * M * 2;
  const unsigned long long t0 = wall_clock64();
  for (;;) {
    if (lane < 2 * STEP_MAX_M) tot_s[lane] = 0ull;
    int cnt = 0;
    for (int idx = lane; idx < nv; idx += 64) {
      const long long v = ld_dev(st + idx);
      cnt += stat_count(v);
      atomicAdd(&tot_s[idx % (2 * M)], stat_sum(v));
    }
    const int rs = (int)row_sum16((float)cnt);
    const int wc = __builtin_amdgcn_readlane(rs, 0) + __builtin_amdgcn_readlane(rs, 16) +
                   __builtin_amdgcn_readlane(rs, 32) + __builtin_amdgcn_readlane(rs, 48);
    if (wc == 2 * M * P.G) return true;
    if (ld_dev(reinterpret_cast<const int*>(P.ws + P.status_off)) != 0) return false;
    if (wall_clock64() - t0 > kTimeoutTicks) {
      set_status(P, MK_ETIMEOUT);
      return false;
    }
    __builtin_amdgcn_s_sleep(8);
  }
}

// End of a phase in one workgroup: add the wave parts of each tile and
// publish the tile's slice partial; then, for the tiles this workgroup
// finishes (tile t is finished by the workgroup of slice t % sk), wait until
// every slice has arrived, add the partials in slice order, apply the
// standardization of the phase input (its row statistics were added up while
// the input was staged) and count the tiles as finished. Spreading the finishing
// over the slices keeps every workgroup's share of it equal.
template <int NM, int MODE>
__device__ __forceinline__ bool phase_outputs(const StepParams& P, const DevPhase& ph, int p,
                                              int l, const DevLayer* ltab, const Assign& a,
                                              int ffirst, int nfin, const char* contrib,
                                              int* abort_s, unsigned long long* wst,
                                              unsigned long long* tot_s, float2* mom_s,
                                              int* cnt_s, int tid) {
  const __amdgpu_buffer_rsrc_t pr = make_rsrc(P.ws + ph.part_off, ph.part_bytes);
  if (tid < 2 * STEP_MAX_M) wst[tid] = 0ull;
  // Every tile's wave parts sit in LDS (slot: tile, wave - first wave of the
  // tile); add them and publish the tile's slice partial. Items (tile,
  // matrix, lane); lanes that hold only rows past M have nothing to publish.
  const int items = a.tw * NM * 64;
  for (int e = tid; e < items; e += STEP_THREADS) {
    const int tl = e / (NM * 64), q = (e >> 6) % NM, ln = e & 63;
    if (4 * (ln >> 4) >= P.M) continue;
    const int tg = a.t0 + tl;
    const int w0 = wave_of_unit(a, tl * a.nkb);
    const int w1 = wave_of_unit(a, (tl + 1) * a.nkb - 1);
    floatx4 v = *reinterpret_cast<const floatx4*>(
        contrib + ((size_t)(tl * ph.cmax) * NM + q) * 1024 + ln * 16);
    for (int kk = 1; kk <= w1 - w0; ++kk) {
      // waves with an empty range (fewer units than waves) wrote nothing
      if (wave_begin(a, w0 + kk) == wave_begin(a, w0 + kk + 1)) continue;
      const floatx4 u = *reinterpret_cast<const floatx4*>(
          contrib + ((size_t)(tl * ph.cmax + kk) * NM + q) * 1024 + ln * 16);
      v += u;
    }
    st4_dev(pr, ((unsigned)(tg * ph.sk + a.s) * NM + q) * 1024u + ln * 16,
            tag_parity(v, (unsigned)l & 1u));
  }
  if (tid == 0) *abort_s = 0;
  // each row's mean and 1/sqrt(var + 1e-6), once (rows past M: zeros)
  if (tid < STEP_MAX_M)
    mom_s[tid] = tid < P.M ? phase_moments(tot_s, tid, ph) : float2{0.f, 0.f};
  __syncthreads();
  tl_stamp(P, l, p, TL_PUBLISHED);
  if (ph.norm != NORM_NONE && (*cnt_s != 2 * P.M * P.G || P.reload)) {  // the same in every thread
    const long long* st = reinterpret_cast<const long long*>(P.ws + P.stats_off) +
                          (size_t)(l * 4 + p) * STAT_SLOTS * P.M * 2;
    if (tid < 64 && !reload_stats(P, st, tot_s, tid)) *abort_s = 1;  // wave 0
    __syncthreads();
    if (*abort_s) return false;
    if (tid < STEP_MAX_M)
      mom_s[tid] = tid < P.M ? phase_moments(tot_s, tid, ph) : float2{0.f, 0.f};
    __syncthreads();
  }
  fixup_tiles<NM, MODE>(P, ph, p, l, ltab, a, ffirst, nfin, wst, mom_s, abort_s, tid);
  wait_vm0();
  __syncthreads();
  tl_stamp(P, l, p, TL_FINISHED);
  if (*abort_s) return false;
  if (tid < nfin) {
    unsigned* done = reinterpret_cast<unsigned*>(P.ws + P.done_off);
    const int tg = a.t0 + ffirst + tid * ph.sk;
    __hip_atomic_fetch_add(done + (size_t)(tg % DONE_CTRS) * CTR_STRIDE, 1u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
  }
  // the next input's statistics: this workgroup's share of each word, after
  // the done counters (a consumer that reads a word before every share is in
  // sees it by the count and reloads at the end of its phase)
  const bool stats = MODE == 0 ? (p < 3 || l + 1 < P.n_layers)
                               : (p == 1 || (p == 3 && l + 1 < P.n_layers));
  if (stats && tid < 2 * P.M) {
    const int ln = p < 3 ? l : l + 1, pn = p < 3 ? p + 1 : 0;
    long long* stl = reinterpret_cast<long long*>(P.ws + P.stats_off) +
                     (size_t)(ln * 4 + pn) * STAT_SLOTS * P.M * 2;
    __hip_atomic_fetch_add(stl + (size_t)(blockIdx.x % STAT_SLOTS) * P.M * 2 + tid,
                           stat_share(wst[tid]), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
  }
  return true;
}

}  // namespace

// MODE 0: the walk of standardized products between binary16 casts; MODE 1:
// the residual walk (RMSNorm with weights, residual adds, SiLU * up). Q6: the
// walk also reads Q6_K walk records (v and down of the layers that have them);
// without it the kernel holds no Q6_K code at all.
template <int MODE, bool Q6, bool TAB>
__global__ void __launch_bounds__(STEP_THREADS) q4k_step_kernel(StepParams P) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  __shared__ DevLayer ltab[STEP_MAX_LAYERS];  // every layer's pointers, read from LDS
  // this workgroup's split of each phase (the same in every layer), each
  // wave's first unit, end unit, tile and super-block, and the first and
  // number of the tiles it finishes
  __shared__ Assign asg[4];
  __shared__ DevPhase ph_s[4];  // LDS copy of the phase table (read with variable indices)
  __shared__ int4 wstart[4][STEP_WAVES];
  __shared__ int4 wseg[4][STEP_WAVES];
  __shared__ int2 fin_s[4];
  __shared__ unsigned long long tot_s[2 * STEP_MAX_M];  // statistics of the phase input
  __shared__ float2 mom_s[STEP_MAX_M];                  // its rows' mean and 1/sigma
  __shared__ unsigned long long wst_s[2 * STEP_MAX_M];  // next input's statistics, being added
  __shared__ int abort_s;
  __shared__ int cnt_s;  // shares counted in the phase input's statistics words when staged
  const int M = P.M;
  const int w = blockIdx.x;
  const int tid = threadIdx.x;
  const int wave = uni(tid >> 6), lane = tid & 63;
  const int c = lane & 15, g = lane >> 4;
  const DevPhase* PH = P.ph;
  const DevLayer* layers = reinterpret_cast<const DevLayer*>(P.ws + P.layers_off);
  {
    const int nw = (int)(sizeof(ph_s) / 4);
    for (int i = tid; i < nw; i += STEP_THREADS)
      reinterpret_cast<uint32_t*>(ph_s)[i] = reinterpret_cast<const uint32_t*>(PH)[i];
  }
  if (tid < 4) {
    const DevPhase& q = PH[tid];
    const Assign x = assign_split(q.nt, q.sk, q.nkb, q.KB, w, P.G);
    asg[tid] = x;
    const int ff = ((x.s - x.t0) % q.sk + q.sk) % q.sk;
    fin_s[tid] = int2{ff, ff < x.tw ? (x.tw - 1 - ff) / q.sk + 1 : 0};
  }
  {
    const uint32_t* lsrc = reinterpret_cast<const uint32_t*>(layers);
    uint32_t* ldst = reinterpret_cast<uint32_t*>(ltab);
    const int nw = P.n_layers * (int)(sizeof(DevLayer) / 4);
    for (int i = tid; i < nw; i += STEP_THREADS) ldst[i] = lsrc[i];
  }
  __syncthreads();
  if (tid < 4 * STEP_WAVES) {
    const int q = tid / STEP_WAVES, v = tid % STEP_WAVES;
    const Assign& x = asg[q];
    const DevPhase& ph = PH[q];
    const int u = wave_begin(x, v), ub = wave_begin(x, v + 1);
    const int tl = x.nkb > 0 ? u / x.nkb : 0;
    const int tg = x.t0 + tl;
    const int seg = (tg >= ph.seg_t0[1]) + (tg >= ph.seg_t0[2]);
    wstart[q][v] = int4{u, ub, tg, u - tl * x.nkb};
    // a wave with no units keeps the phase's first matrix (never read)
    // (the record index; its size depends on the matrix's type in each layer)
    wseg[q][v] = u < ub ? int4{ph.mat0 + seg,
                               (int)((unsigned)(tg - ph.seg_t0[seg]) * (unsigned)ph.KB +
                                     (unsigned)x.kb0),
                               ph.seg_t0[seg + 1], 0}
                        : int4{ph.mat0, 0, ph.nt, 0};
  }
  if (tid < 2 * STEP_MAX_M) {
    wst_s[tid] = 0ull;
    tot_s[tid] = 0ull;
  }
  if (tid == 0) cnt_s = 0;
  __syncthreads();
  const UnpackConsts k = unpack_consts(g);
  // Rows past M read row M-1 (their results are never stored), so every
  // lane's activation reads are unconditional.
  const int arow = c < M ? c : M - 1;

  BlockRegs ring[STEP_PD];
  Iter it;
  RecTab tb = {0u, 0u, 0u};
  Assign a = lds_assign(asg[0]);
  if constexpr (TAB) {
    tb = build_tab<Q6>(ph_s[0], &ltab[0], a, wave, lane);
    ring_fill_tab<Q6>(ring, tb, ph_s[0], &ltab[0], a, wave, lane);
  } else {
    iter_init<Q6>(it, ph_s[0], &ltab[0], wstart[0][wave], wseg[0][wave]);
    ring_fill<Q6>(ring, it, ph_s[0], &ltab[0], a, lane);
  }

  // ---- layer-0 input: this workgroup's columns of it (MODE 0: a copy of
  //      x0; MODE 1: the cast of h0 times the first norm weight) and their
  //      row sums, added to its statistics
  {
    const int c0 = (int)((long long)P.H * w / P.G), c1 = (int)((long long)P.H * (w + 1) / P.G);
    const int nc = c1 - c0;
    const __amdgpu_buffer_rsrc_t x0r = make_rsrc(ltab[0].x[0], (unsigned)(M * P.H * 2));
    for (int i = tid; i < M * nc; i += STEP_THREADS) {
      const int m = i / nc, cc = c0 + (i - m * nc);
      if (MODE == 0) {
        const uint16_t hb = to_global(P.x0)[(size_t)m * P.H + cc];
        to_global(ltab[0].x[0])[(size_t)m * P.H + cc] = hb;
        const float h = (float)bit_cast_<_Float16>(hb);
        atomicAdd(&wst_s[2 * m], (unsigned long long)round_i64((double)h * STAT_SCALE_SUM));
        atomicAdd(&wst_s[2 * m + 1],
                  (unsigned long long)round_i64((double)(h * h) * STAT_SCALE_SQ));
      } else {
        const float hv = to_global(P.h0)[(size_t)m * P.H + cc];
        float v = hv * to_global(ltab[0].g[0])[cc];
        asm volatile("" : "+v"(v));
        const uint16_t hb = bit_cast_<uint16_t>((_Float16)v);
        // read by other workgroups after the start barrier: device-coherent
        __builtin_amdgcn_raw_buffer_store_b16(hb, x0r, (unsigned)((m * P.H + cc) * 2), 0,
                                              kCoherent);
        const double sq = (double)hv * (double)hv;
        if ((hb & 0x7C00) == 0x7C00 || !(sq < RMS_TERM_MAX)) {
          set_status(P, MK_ERANGE);
        } else {
          const double t = __builtin_rint(sq * RMS_SCALE);
          const double hi = __builtin_floor(t * (1.0 / 4294967296.0));
          atomicAdd(&wst_s[2 * m], (unsigned long long)(long long)hi);
          atomicAdd(&wst_s[2 * m + 1],
                    (unsigned long long)(long long)__builtin_fma(-hi, 4294967296.0, t));
        }
      }
    }
    __syncthreads();
    if (tid < 2 * M) {
      long long* st0 = reinterpret_cast<long long*>(P.ws + P.stats_off);
      const long long v = (long long)wst_s[tid];
      if (MODE == 0 && !(fabs((double)v) < STAT_TERM_MAX)) set_status(P, MK_ERANGE);
      __hip_atomic_fetch_add(st0 + (size_t)(w % STAT_SLOTS) * M * 2 + tid,
                             stat_share((unsigned long long)v), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
    }
    wait_vm0();
    __syncthreads();
    if (tid == 0)
      __hip_atomic_fetch_add(reinterpret_cast<unsigned*>(P.ws + P.start_off), 1u,
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // every workgroup's share must be in before the first staging reads the
    // statistics
    if (tid == 0) abort_s = 0;
    if (!wait_start(P, &abort_s)) return;
  }

  for (int l = 0; l < P.n_layers; ++l) {
    const DevLayer* L = &ltab[l];
    for (int p = 0; p < 4; ++p) {
      const DevPhase& ph = PH[p];
      char* x_lds = smem;
      char* xs_lds = x_lds + (size_t)M * ph.x_stride;
      char* contrib = smem + ph.lds_contrib;
      // ---- stage this phase's binary16 input slice (the first weight
      //      records are already in flight); MODE 0 reads layer 0's from x0
      stage_slice(MODE == 0 && l == 0 && p == 0 ? P.x0 : L->x[p], ph.K, M, a,
                  reinterpret_cast<const long long*>(P.ws + P.stats_off) +
                      (size_t)(l * 4 + p) * STAT_SLOTS * M * 2,
                  tot_s, x_lds, ph.x_stride, xs_lds, xsum_row_bytes(ph.nkb), &cnt_s, tid);
      __syncthreads();
      tl_stamp(P, l, p, TL_START);

      // ---- stream the weights
      const char* xa_lane = x_lds + (size_t)arow * ph.x_stride + g * 128;
      const char* xs_lane = xs_lds + (size_t)arow * xsum_row_bytes(ph.nkb) + 16 * g;
      if constexpr (TAB) {
        if (ph.nm == 2)
          phase_compute_tab<2, Q6>(ring, tb, ph_s[p], &ltab[l], a, wave, lane, xa_lane, xs_lane,
                                   contrib, k);
        else
          phase_compute_tab<1, Q6>(ring, tb, ph_s[p], &ltab[l], a, wave, lane, xa_lane, xs_lane,
                                   contrib, k);
      } else {
        if (ph.nm == 2)
          phase_compute<2, Q6>(ring, it, ph_s[p], &ltab[l], a, wave, lane, xa_lane, xs_lane,
                               contrib, k);
        else
          phase_compute<1, Q6>(ring, it, ph_s[p], &ltab[l], a, wave, lane, xa_lane, xs_lane,
                               contrib, k);
      }
      __syncthreads();
      tl_stamp(P, l, p, TL_COMPUTED);

      // ---- finish tiles, start the next phase's weight stream, wait until
      //      every tile of this phase is finished
      const int ffirst = uni(fin_s[p].x), nfin = uni(fin_s[p].y);
      const bool ok = ph.nm == 2
                          ? phase_outputs<2, MODE>(P, ph, p, l, ltab, a, ffirst, nfin, contrib, &abort_s,
                                             wst_s, tot_s, mom_s, &cnt_s, tid)
                          : phase_outputs<1, MODE>(P, ph, p, l, ltab, a, ffirst, nfin, contrib, &abort_s,
                                             wst_s, tot_s, mom_s, &cnt_s, tid);
      if (!ok) return;
      // the next staging adds the next input's statistics from zero (ordered
      // before its atomics by the barrier that ends wait_done)
      if (tid < 2 * STEP_MAX_M) tot_s[tid] = 0ull;
      if (tid == 0) cnt_s = 0;
      const int ln = p < 3 ? l : l + 1, pn = p < 3 ? p + 1 : 0;
      if (ln < P.n_layers) {
        a = lds_assign(asg[pn]);
        if constexpr (TAB) {
          tb = build_tab<Q6>(ph_s[pn], &ltab[ln], a, wave, lane);
          ring_fill_tab<Q6>(ring, tb, ph_s[pn], &ltab[ln], a, wave, lane);
        } else {
          iter_init<Q6>(it, ph_s[pn], &ltab[ln], wstart[pn][wave], wseg[pn][wave]);
          ring_fill<Q6>(ring, it, ph_s[pn], &ltab[ln], a, lane);
        }
      }
      if (!wait_done(P, PH, l, p, &abort_s)) return;
      tl_stamp(P, l, p, TL_DONE_SEEN);
    }
  }

  // x_out was written by the finishers of the last layer's down projection
}

// Zero the counters, status word and statistics, and fill every slice
// partial piece with words of parity 1 (not yet written in layer 0).
__global__ void __launch_bounds__(256) q4k_step_clear(uint32_t* p, size_t n, uint32_t* part,
                                                      size_t npart, size_t keep0, size_t keep1) {
  // words [keep0, keep1) keep their value (a later row group keeps the status)
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    if (i < keep0 || i >= keep1) p[i] = 0u;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < npart;
       i += (size_t)gridDim.x * blockDim.x)
    part[i] = PART_FILL;
}

}  // namespace mk

// ----------------------------------------------------------------- host side
namespace mk {

namespace {

constexpr int kMaxG = 1024;                    // most workgroups (CUs) planned for
std::atomic<int> g_walk_form{MK_WALK_AUTO};     // mk_q4k_step_set_walk_form
constexpr size_t kLdsLimit = 160 * 1024;
// the kernel's static LDS arrays (layer and phase tables, work splits,
// statistics), with room for alignment
constexpr size_t kStaticLds = 4 * sizeof(Assign) + 4 * sizeof(DevPhase) +
                              2 * 4 * STEP_WAVES * 16 + 4 * 8 +
                              STEP_MAX_LAYERS * sizeof(DevLayer) +
                              STEP_MAX_M * sizeof(float) * 2 +
                              2 * 2 * STEP_MAX_M * sizeof(unsigned long long) + 256;

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

int tiles_of(int n) { return (n + 15) / 16; }

struct StepPlan {
  DevPhase ph[4];
  size_t layers_off, done_off, status_off, start_off, stats_off, sync_end;
  size_t part_begin, part_end;  // slice partial blocks of all phases
  size_t tl_off;                // MK_STEP_TIMELINE: the stamps (0 otherwise)
  size_t total;
  bool ok = true;  // false: some K slice would get no workgroup
  bool tab = false;  // every phase's waves fit a record table (DevPhase::tab)
  bool reload = false;  // MK_WALK_RELOAD_STATS: every phase reloads its input statistics
};

// Host mirror of the device work split (the same shared functions).
void host_assign(const DevPhase& ph, int w, int G, int* t0, int* tw, int* nkb) {
  const Assign a = assign_split(ph.nt, ph.sk, ph.nkb, ph.KB, w, G);
  *t0 = a.t0;
  *tw = a.tw;
  *nkb = a.nkb;
}

int host_wave_of_unit(int U, int x) {
  Assign a = {};
  a.U = U;
  return wave_of_unit(a, x);
}

// Fill the phase table for the shapes of layer 0; sk is chosen so that one
// slice of staged activations fits the LDS budget. Offsets are relative to
// the workspace base. G only enters tw_max (LDS sizing).
void plan_phases(const mk_q4k_layer& L0, int n_layers, int M, int G, StepPlan& sp) {
  const mk_q4k_mat* mats[7] = {&L0.q, &L0.k, &L0.v, &L0.o, &L0.gate, &L0.up, &L0.down};
  memset(&sp, 0, sizeof(sp));
  sp.ok = true;
  for (int p = 0; p < 4; ++p) {
    DevPhase& ph = sp.ph[p];
    int first, nseg;
    switch (p) {
      case 0: first = 0; nseg = 3; ph.nm = 1; break;
      case 1: first = 3; nseg = 1; ph.nm = 1; break;
      case 2: first = 4; nseg = 1; ph.nm = 2; break;
      default: first = 6; nseg = 1; ph.nm = 1; break;
    }
    ph.mat0 = first;
    ph.nseg = nseg;
    ph.K = mats[first]->K;
    ph.KB = ph.K / QK;
    ph.inv_k = 1.0 / ph.K;
    int t = 0, c = 0;
    for (int s = 0; s < 3; ++s) {
      if (s < nseg) {
        ph.seg_n[s] = mats[first + s]->N;
        ph.seg_t0[s] = t;
        ph.seg_c0[s] = c;
        t += tiles_of(ph.seg_n[s]);
        c += ph.seg_n[s] * ph.nm;
      } else {
        ph.seg_n[s] = 1;
        ph.seg_t0[s] = t;
        ph.seg_c0[s] = c;
      }
    }
    ph.seg_t0[3] = t;
    for (int s = nseg; s < 3; ++s) ph.seg_t0[s] = t;
    ph.nt = t;
    ph.ncols = c;
    // column sums of segment s's matrix: after its tile records
    for (int s = 0; s < 3; ++s) {
      ph.cs_off[s] = s < nseg ? (unsigned)((size_t)tiles_of(ph.seg_n[s]) * ph.KB * TILE_REC) : 0u;
      ph.cs_off6[s] = s < nseg ? (unsigned)((size_t)tiles_of(ph.seg_n[s]) * ph.KB * Q6W_REC) : 0u;
    }
    // K slices: at least 4, more while one slice of activations of the most
    // rows the walk takes (STEP_MAX_M, whatever M is: the slices, and so every
    // summation order, do not depend on the row count, and a row's results
    // are the same, bit for bit, alone or stacked) exceeds 96 KiB of LDS or
    // takes more than one round of loads to stage
    const int Mp = STEP_MAX_M;
    int sk = 4 < ph.KB ? 4 : ph.KB;
    for (;;) {
      int nkb = (ph.KB + sk - 1) / sk;
      size_t xb = (size_t)Mp * (nkb * X_BYTES_PER_BLOCK + X_ROW_PAD) +
                  (size_t)Mp * xsum_row_bytes(nkb);
      const bool one_round = Mp * nkb * 32 <= STEP_THREADS * kStageRound;
      if ((xb <= 96 * 1024 && one_round) || nkb == 1) {
        ph.sk = (ph.KB + nkb - 1) / nkb;
        ph.nkb = nkb;
        break;
      }
      ++sk;
    }
    ph.x_stride = ph.nkb * X_BYTES_PER_BLOCK + X_ROW_PAD;
    if (M * ph.nkb * 32 > STEP_THREADS * kStageRound) sp.ok = false;  // staging is one round
    for (int q = 0; q < ph.sk; ++q)
      if (slice_start(q + 1, ph.sk, ph.nkb, ph.KB, G) <= slice_start(q, ph.sk, ph.nkb, ph.KB, G))
        sp.ok = false;
    ph.tw_max = 0;
    ph.cmax = 1;
    for (int w = 0; w < G; ++w) {
      int t0, tw, nkb;
      host_assign(ph, w, G, &t0, &tw, &nkb);
      if (tw > ph.tw_max) ph.tw_max = tw;
      const int U = tw * nkb;
      for (int tl = 0; tl < tw; ++tl) {
        const int c = host_wave_of_unit(U, (tl + 1) * nkb - 1) - host_wave_of_unit(U, tl * nkb) + 1;
        if (c > ph.cmax) ph.cmax = c;
      }
    }
    if (ph.tw_max < 1) ph.tw_max = 1;
    // the record table holds up to TAB_MAX records of a wave, and a unit's
    // super-block in 4 bits
    {
      int maxrec = 0;
      for (int w = 0; w < G; ++w) {
        const Assign a = assign_split(ph.nt, ph.sk, ph.nkb, ph.KB, w, G);
        for (int v = 0; v < SPLIT_WAVES; ++v) {
          const int r = (wave_begin(a, v + 1) - wave_begin(a, v)) * ph.nm;
          if (r > maxrec) maxrec = r;
        }
      }
      ph.tab = maxrec <= TAB_MAX && ph.nkb <= 15 ? 1 : 0;
    }
    {
      const size_t xb = (size_t)M * ph.x_stride + (size_t)M * xsum_row_bytes(ph.nkb);
      const size_t c0 = (xb + 15) & ~(size_t)15;
      ph.lds_contrib = (int)c0;
      ph.lds_bytes = (int)(c0 + (size_t)ph.tw_max * ph.cmax * ph.nm * 1024);
    }
  }
  // workspace layout
  size_t off = 0;
  sp.done_off = off;
  off += align256((size_t)DONE_CTRS * CTR_STRIDE * sizeof(unsigned));
  sp.status_off = off;
  off += 256;
  sp.start_off = off;
  off += 256;
  sp.stats_off = off;
  off += align256((size_t)n_layers * 4 * STAT_SLOTS * M * 2 * sizeof(long long));
  sp.sync_end = off;
  sp.layers_off = off;  // one layer table per row group
  off += align256((size_t)STEP_GROUPS * n_layers * sizeof(DevLayer));
  sp.tab = sp.ph[0].tab && sp.ph[1].tab && sp.ph[2].tab && sp.ph[3].tab;
  // each statistics slot's sum stays below 2^58 (STAT_SLOT_TERMS terms of
  // at most 2^50): the slot's workgroups times the tiles one finishes, and
  // times the layer-0 input columns one adds up (RMS terms, one per value)
  {
    const int per_slot = (G + STAT_SLOTS - 1) / STAT_SLOTS;
    for (int p = 0; p < 4; ++p) {
      const int nfin = (sp.ph[p].tw_max + sp.ph[p].sk - 1) / sp.ph[p].sk;
      if ((long long)per_slot * nfin > STAT_SLOT_TERMS) sp.ok = false;
    }
    const int H = L0.q.K;
    if ((long long)per_slot * ((H + G - 1) / G) > STAT_SLOT_TERMS) sp.ok = false;
  }
  sp.part_begin = off;
  for (int p = 0; p < 4; ++p) {
    sp.ph[p].part_off = off;
    const size_t pb = (size_t)sp.ph[p].nt * sp.ph[p].sk * sp.ph[p].nm * 1024;
    sp.ph[p].part_bytes = (unsigned)pb;
    off += align256(pb);
  }
  sp.part_end = off;
  sp.tl_off = 0;
  if (MK_STEP_TIMELINE) {
    sp.tl_off = off;
    off += align256((size_t)n_layers * 4 * kMaxG * TL_EVENTS * sizeof(unsigned long long));
  }
  sp.total = off;
}

size_t lds_bytes(const StepPlan& sp, int) {
  size_t mx = 0;
  for (int p = 0; p < 4; ++p)
    if ((size_t)sp.ph[p].lds_bytes > mx) mx = (size_t)sp.ph[p].lds_bytes;
  return mx;
}

bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_mat(const mk_q4k_mat& m) {
  if (m.N < 1 || m.K < QK || m.K % QK) return MK_EINVAL;
  // record offsets within one matrix are 32-bit
  if ((size_t)tiles_of(m.N) * (size_t)(m.K / QK) * TILE_REC >= ((size_t)1 << 32)) return MK_EINVAL;
  return MK_OK;
}

bool same_shape(const mk_q4k_mat& a, const mk_q4k_mat& b) { return a.N == b.N && a.K == b.K; }

int check_step_shapes(const mk_q4k_layer* layers, int n_layers, int M) {
  if (!layers || n_layers < 1 || n_layers > STEP_MAX_LAYERS || M < 1 || M > STEP_MAX_ROWS)
    return MK_EINVAL;
  const mk_q4k_layer& L = layers[0];
  const mk_q4k_mat* m[7] = {&L.q, &L.k, &L.v, &L.o, &L.gate, &L.up, &L.down};
  for (int i = 0; i < 7; ++i)
    if (check_mat(*m[i]) != MK_OK) return MK_EINVAL;
  const int H = L.q.K;
  if (L.k.K != H || L.v.K != H || L.gate.K != H || L.up.K != H || L.down.N != H) return MK_EINVAL;
  if (L.o.K != L.q.N) return MK_EINVAL;
  if (L.gate.N != L.up.N || L.down.K != L.gate.N) return MK_EINVAL;
  if (L.o.N != H) return MK_EINVAL;
  for (int l = 1; l < n_layers; ++l) {
    const mk_q4k_layer& B = layers[l];
    if (!same_shape(B.q, L.q) || !same_shape(B.k, L.k) || !same_shape(B.v, L.v) ||
        !same_shape(B.o, L.o) || !same_shape(B.gate, L.gate) || !same_shape(B.up, L.up) ||
        !same_shape(B.down, L.down))
      return MK_EINVAL;
  }
  // block types: Q4_K everywhere, Q6_K allowed for v and down (Q4_K_M files)
  for (int l = 0; l < n_layers; ++l) {
    const mk_q4k_layer& B = layers[l];
    const mk_q4k_mat* q4[5] = {&B.q, &B.k, &B.o, &B.gate, &B.up};
    for (int i = 0; i < 5; ++i)
      if (q4[i]->type != 0 && q4[i]->type != MK_QTYPE_Q4_K) return MK_EINVAL;
    const mk_q4k_mat* q6[2] = {&B.v, &B.down};
    for (int i = 0; i < 2; ++i)
      if (q6[i]->type != 0 && q6[i]->type != MK_QTYPE_Q4_K && q6[i]->type != MK_QTYPE_Q6_K)
        return MK_EINVAL;
  }
  return MK_OK;
}

// Last layer table copied into each workspace, to skip identical re-copies.
struct TableCache {
  const void* ws = nullptr;
  std::vector<DevLayer> table;
  DevPhase phases[4];
};
TableCache g_table_cache[64][STEP_GROUPS];  // per device and row group
std::mutex g_table_mu;

// The part of a step call both walks share: plan, checks, the device layer
// table (re-sent only when it changed), the clear kernel and the launch.
// Plan of a walk over M rows (a row group), with the checks made before any
// work is enqueued: the split, the workspace size, the LDS and occupancy.
// The kernel of a walk: with the Q6_K path or not, and with the record tables
// (every wave of every phase fits one) or the record iterator.
template <int MODE>
const void* walk_kernel(bool q6, bool tab) {
  if (tab)
    return q6 ? (const void*)q4k_step_kernel<MODE, true, true>
              : (const void*)q4k_step_kernel<MODE, false, true>;
  return q6 ? (const void*)q4k_step_kernel<MODE, true, false>
            : (const void*)q4k_step_kernel<MODE, false, false>;
}

template <int MODE>
int prepare_walk(const mk_q4k_layer* layers, int n_layers, int M, size_t ws_bytes, bool q6,
                 StepPlan& sp, size_t& lds, int& G) {
  int cus = 0;
  const int rc = current_gfx950(&cus);
  if (rc != MK_OK) return rc;
  G = cus < kMaxG ? cus : kMaxG;
  plan_phases(layers[0], n_layers, M, G, sp);
  if (!sp.ok) return MK_EINVAL;
  const int form = g_walk_form.load(std::memory_order_relaxed);
  if (form & MK_WALK_ITERATOR) sp.tab = false;
  sp.reload = (form & MK_WALK_RELOAD_STATS) != 0;
  for (int p = 0; p < 4; ++p)
    sp.ph[p].norm = MODE == 0 ? NORM_STD : (p == 0 || p == 2 ? NORM_RMS : NORM_NONE);
  if (ws_bytes < sp.total) return MK_EWORKSPACE;
  for (int p = 0; p < 4; ++p) {
    if (sp.ph[p].sk > G) return MK_EINVAL;
    // partial blocks are addressed with 32-bit buffer offsets
    if ((size_t)sp.ph[p].nt * sp.ph[p].sk * sp.ph[p].nm * 1024 >= (1ull << 32)) return MK_EINVAL;
  }
  lds = lds_bytes(sp, M);
  if (lds + kStaticLds > kLdsLimit) return MK_EINVAL;
  hipError_t e = hipFuncSetAttribute(walk_kernel<MODE>(q6, sp.tab),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return MK_EHIP;
  int occ = 0;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, walk_kernel<MODE>(q6, sp.tab), STEP_THREADS,
                                                    lds);
  if (e != hipSuccess) return MK_EHIP;
  if (occ < 1) return MK_EOCCUPANCY;
  return MK_OK;
}

// Enqueue one walk (row group `group` of the call, M rows) on the stream:
// its layer table (copied only when it changed), the clear of the
// synchronisation words (a later group keeps the status word, so the call
// reports the first failure of any group) and the persistent kernel.
template <int MODE>
int enqueue_walk(const mk_q4k_layer* layers, const std::vector<DevLayer>& table, int n_layers,
                 int M, const uint16_t* x0, uint16_t* x_out, const float* h0, void* workspace,
                 const StepPlan& sp, size_t lds, int G, int group, bool q6, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  const size_t table_off = sp.layers_off + (size_t)group * n_layers * sizeof(DevLayer);
  hipError_t e;
  {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return MK_EHIP;
    std::lock_guard<std::mutex> lk(g_table_mu);
    TableCache& tc = g_table_cache[dev][group];
    const bool same = tc.ws == workspace && tc.table.size() == table.size() &&
                      memcmp(tc.table.data(), table.data(), table.size() * sizeof(DevLayer)) == 0 &&
                      memcmp(tc.phases, sp.ph, sizeof(sp.ph)) == 0;
    if (!same) {
      // pageable sources: the calls return once the host buffers have been read
      e = hipMemcpyAsync(ws + table_off, table.data(), table.size() * sizeof(DevLayer),
                         hipMemcpyHostToDevice, st);
      if (e != hipSuccess) return MK_EHIP;
      tc.ws = workspace;
      tc.table = table;
      memcpy(tc.phases, sp.ph, sizeof(sp.ph));
    }
  }
  // clear flags, status, counters and statistics
  const size_t nclear = sp.sync_end / sizeof(uint32_t);
  const size_t keep0 = group > 0 ? sp.status_off / sizeof(uint32_t) : 0;
  const size_t keep1 = group > 0 ? keep0 + 1 : 0;
  hipLaunchKernelGGL(q4k_step_clear, dim3(256), dim3(256), 0, st,
                     reinterpret_cast<uint32_t*>(ws), nclear,
                     reinterpret_cast<uint32_t*>(ws + sp.part_begin),
                     (sp.part_end - sp.part_begin) / sizeof(uint32_t), keep0, keep1);
  e = hipGetLastError();
  if (e != hipSuccess) return MK_EHIP;

  StepParams P;
  memset(&P, 0, sizeof(P));
  memcpy(P.ph, sp.ph, sizeof(sp.ph));
  P.n_layers = n_layers;
  P.M = M;
  P.G = G;
  P.H = layers[0].q.K;
  P.x0 = x0;
  P.x_out = x_out;
  P.h0 = h0;
  P.ws = ws;
  P.layers_off = table_off;
  P.done_off = sp.done_off;
  P.stats_off = sp.stats_off;
  P.start_off = sp.start_off;
  P.status_off = sp.status_off;
  P.lds_bytes = lds;
  P.tl_off = sp.tl_off;
  P.reload = sp.reload ? 1 : 0;
  const void* kern = walk_kernel<MODE>(q6, sp.tab);
  void* args[] = {&P};
  e = hipLaunchKernel(kern, dim3(G), dim3(STEP_THREADS), args, lds, st);
  if (e != hipSuccess) return MK_EHIP;
  e = hipGetLastError();
  return e == hipSuccess ? MK_OK : MK_EHIP;
}

// Whether any matrix of the walk is Q6_K (then the kernel built for it runs).
bool any_q6(const mk_q4k_layer* layers, int n_layers) {
  for (int l = 0; l < n_layers; ++l)
    if (layers[l].v.type == MK_QTYPE_Q6_K || layers[l].down.type == MK_QTYPE_Q6_K) return true;
  return false;
}

// Rows [r0, r0 + STEP_MAX_M) of the call: row group r0 / STEP_MAX_M.
int group_rows(int M, int g) {
  const int r = M - g * STEP_MAX_M;
  return r < STEP_MAX_M ? r : STEP_MAX_M;
}

// Host-side checks of the per-layer weights and outputs both walks share.
int check_layer_io(const mk_q4k_layer* layers, float* const* y, uint16_t* const* x, int l) {
  const mk_q4k_layer& L = layers[l];
  const void* w[7] = {L.q.w, L.k.w, L.v.w, L.o.w, L.gate.w, L.up.w, L.down.w};
  for (int i = 0; i < 7; ++i) {
    if (!w[i] || !y[i]) return MK_EINVAL;
    if (!al16(w[i]) || !al16(y[i])) return MK_EALIGN;
  }
  for (int i = 0; i < 4; ++i) {
    if (!x[i]) return MK_EINVAL;
    if (!al16(x[i])) return MK_EALIGN;
  }
  return MK_OK;
}

// A layer's table entry for the rows from r0 on: every [M][width] buffer
// starts r0 rows in (outputs [M][N]; inputs x[0], x[2] [M][H], x[1] [M][q.N],
// x[3] [M][gate.N]).
void fill_table(const mk_q4k_layer& L, float* const* y, uint16_t* const* x, int r0, DevLayer& t) {
  const mk_q4k_mat* m[7] = {&L.q, &L.k, &L.v, &L.o, &L.gate, &L.up, &L.down};
  const int xw[4] = {L.q.K, L.q.N, L.gate.K, L.gate.N};
  memset(&t, 0, sizeof(t));
  for (int i = 0; i < 7; ++i) {
    t.w[i] = static_cast<const uint8_t*>(m[i]->w);
    t.y[i] = y[i] + (size_t)r0 * m[i]->N;
    if (m[i]->type == MK_QTYPE_Q6_K) t.q6 |= 1u << i;
  }
  for (int i = 0; i < 4; ++i) t.x[i] = x[i] + (size_t)r0 * xw[i];
}


// Host walk of everything the kernel indexes for one plan, with the kernel's
// own work-split functions (assign_split, wave_begin, wave_of_unit) and the
// record order of its iterator: every weight record, column sum, slice
// partial, LDS slot, staged element, output element and statistics slot each
// workgroup and wave touches must lie inside its buffer. Returns the number
// of accesses that do not.
long long plan_violations(const mk_q4k_layer& L0, int n_layers, int M, int G) {
  StepPlan sp;
  plan_phases(L0, n_layers, M, G, sp);
  const size_t lds = lds_bytes(sp, M);
  // plans the launch refuses (MK_EINVAL) are not walked
  if (!sp.ok || lds + kStaticLds > kLdsLimit) return -1;
  const mk_q4k_mat* mats[7] = {&L0.q, &L0.k, &L0.v, &L0.o, &L0.gate, &L0.up, &L0.down};
  long long bad = 0;
  auto check = [&](bool ok) { bad += ok ? 0 : 1; };
  for (int p = 0; p < 4; ++p) {
    const DevPhase& ph = sp.ph[p];
    check(ph.sk <= G);
    check((size_t)ph.part_bytes == (size_t)ph.nt * ph.sk * ph.nm * 1024);
    // the next phase's input width (the finishers' binary16 stores)
    const int Kn = ph.seg_n[0];
    for (int w = 0; w < G; ++w) {
      const Assign a = assign_split(ph.nt, ph.sk, ph.nkb, ph.KB, w, G);
      check(a.s >= 0 && a.s < ph.sk && a.t0 >= 0 && a.t0 + a.tw <= ph.nt && a.tw <= ph.tw_max);
      check(a.kb0 >= 0 && a.kb0 + a.nkb <= ph.KB && a.nkb >= 1);
      // staging: rows m < M, columns of the slice, LDS rows of x_stride bytes
      check((size_t)(a.kb0 + a.nkb) * QK <= (size_t)ph.K);
      check((size_t)M * ph.x_stride + (size_t)M * xsum_row_bytes(ph.nkb) <=
            (size_t)ph.lds_contrib);
      check((size_t)(a.nkb - 1) * X_BYTES_PER_BLOCK + 3 * 128 + 7 * 16 + 16 <=
            (size_t)ph.x_stride);
      for (int v = 0; v < SPLIT_WAVES; ++v) {
        const int ua = wave_begin(a, v), ub = wave_begin(a, v + 1);
        check(ua >= 0 && ua <= ub && ub <= a.U);
        // a record table holds the wave's records and units, a unit's
        // super-block in 4 bits and its slot offset in 24
        if (ph.tab)
          check((ub - ua) * ph.nm <= TAB_MAX && a.nkb <= 15 &&
                (size_t)ph.tw_max * ph.cmax * ph.nm * 1024 < ((size_t)1 << 24));
        // every record the wave loads (the walk never moves past ub - 1)
        for (int u = ua; u < ub; ++u) {
          const int tl = u / a.nkb, b = u % a.nkb, tg = a.t0 + tl;
          const int seg = (tg >= ph.seg_t0[1]) + (tg >= ph.seg_t0[2]);
          check(seg < ph.nseg && tg >= ph.seg_t0[seg] && tg < ph.seg_t0[seg + 1]);
          for (int q = 0; q < ph.nm; ++q) {
            const mk_q4k_mat& m = *mats[ph.mat0 + seg + q];
            const size_t rec = ((size_t)(tg - ph.seg_t0[seg]) * ph.KB + a.kb0 + b) * TILE_REC;
            check(rec + TILE_REC <= (size_t)tiles_of(m.N) * (m.K / QK) * TILE_REC);
          }
          // the LDS contribution slot of the tile's part
          const int first = wave_of_unit(a, tl * a.nkb);
          check(v >= first && v - first < ph.cmax);
          const size_t slot = ((size_t)(tl * ph.cmax + (v - first)) * ph.nm + ph.nm - 1) * 1024 + 63 * 16;
          check(slot + 16 <= (size_t)ph.tw_max * ph.cmax * ph.nm * 1024 &&
                ph.lds_contrib + slot + 16 <= lds);
        }
      }
      // published slice partials of the workgroup's tiles
      for (int tl = 0; tl < a.tw; ++tl)
        check(((size_t)((a.t0 + tl) * ph.sk + a.s) * ph.nm + ph.nm) * 1024 <= ph.part_bytes);
      // the tiles it finishes: tile t belongs to the workgroup of slice t % sk
      const int ff = ((a.s - a.t0) % ph.sk + ph.sk) % ph.sk;
      const int nfin = ff < a.tw ? (a.tw - 1 - ff) / ph.sk + 1 : 0;
      for (int i = 0; i < nfin; ++i) {
        const int tg = a.t0 + ff + i * ph.sk;
        check(tg < a.t0 + a.tw && tg % ph.sk == a.s);
        check(((size_t)(tg * ph.sk + ph.sk - 1) * ph.nm + ph.nm) * 1024 <= ph.part_bytes);
        const int seg = (tg >= ph.seg_t0[1]) + (tg >= ph.seg_t0[2]);
        const int cs_max = (tg - ph.seg_t0[seg]) * 16 + 15;
        // column sums after the records; outputs and next inputs only below N
        check(cs_max < tiles_of(ph.seg_n[seg]) * 16);
        check(ph.cs_off[seg] ==
              (unsigned)((size_t)tiles_of(ph.seg_n[seg]) * ph.KB * TILE_REC));
        // the same matrix in the Q6_K walk-record form (v, down)
        check(ph.cs_off6[seg] ==
              (unsigned)((size_t)tiles_of(ph.seg_n[seg]) * ph.KB * Q6W_REC));
        check(seg > 0 || ph.seg_n[0] <= Kn);
      }
    }
    // every tile has exactly one finisher
    std::vector<int> fin(ph.nt, 0);
    for (int w = 0; w < G; ++w) {
      const Assign a = assign_split(ph.nt, ph.sk, ph.nkb, ph.KB, w, G);
      const int ff = ((a.s - a.t0) % ph.sk + ph.sk) % ph.sk;
      for (int tg = a.t0 + ff; tg < a.t0 + a.tw; tg += ph.sk) ++fin[tg];
    }
    for (int t = 0; t < ph.nt; ++t) check(fin[t] == 1);
    // every (tile, slice) unit range is covered by exactly one workgroup
    std::vector<int> cover((size_t)ph.nt * ph.sk, 0);
    for (int w = 0; w < G; ++w) {
      const Assign a = assign_split(ph.nt, ph.sk, ph.nkb, ph.KB, w, G);
      for (int tl = 0; tl < a.tw; ++tl) ++cover[(size_t)(a.t0 + tl) * ph.sk + a.s];
    }
    for (size_t i = 0; i < cover.size(); ++i) check(cover[i] == 1);
  }
  check(sp.tab == (sp.ph[0].tab && sp.ph[1].tab && sp.ph[2].tab && sp.ph[3].tab));
  // statistics slots of every (layer, phase) input, and the layer table
  check(sp.stats_off + (size_t)n_layers * 4 * STAT_SLOTS * M * 2 * sizeof(long long) <= sp.sync_end);
  check(sp.layers_off + (size_t)STEP_GROUPS * n_layers * sizeof(DevLayer) <= sp.part_begin);
  return bad;
}

}  // namespace

}  // namespace mk

extern "C" {

long long mk_q4k_step_timeline_offset(const mk_q4k_layer* layer0, int n_layers, int M) {
  if (!MK_STEP_TIMELINE) return -1;
  if (mk::check_step_shapes(layer0, 1, M) != MK_OK || n_layers < 1) return MK_EINVAL;
  mk::StepPlan sp;
  mk::plan_phases(*layer0, n_layers, mk::group_rows(M, 0), mk::kMaxG, sp);
  return sp.ok ? (long long)sp.tl_off : -1;
}

int mk_q4k_step_set_walk_form(int form) {
  if ((form & ~(MK_WALK_ITERATOR | MK_WALK_RELOAD_STATS)) != 0) return MK_EINVAL;
  mk::g_walk_form.store(form, std::memory_order_relaxed);
  return MK_OK;
}

long long mk_q4k_step_check_plan(const mk_q4k_layer* layer0, int n_layers, int M, int G) {
  if (mk::check_step_shapes(layer0, 1, M) != MK_OK || n_layers < 1 ||
      n_layers > mk::STEP_MAX_LAYERS || G < 1 || G > mk::kMaxG)
    return MK_EINVAL;
  // the first row group and the last (the only one that can be smaller)
  const int last = (M - 1) / mk::STEP_MAX_M;
  long long bad = mk::plan_violations(*layer0, n_layers, mk::group_rows(M, 0), G);
  if (bad >= 0 && last > 0) {
    const long long b2 = mk::plan_violations(*layer0, n_layers, mk::group_rows(M, last), G);
    bad = b2 < 0 ? b2 : bad + b2;
  }
  return bad;
}


size_t mk_q4k_step_workspace_bytes(const mk_q4k_layer* layer0, int n_layers, int M) {
  if (mk::check_step_shapes(layer0, 1, M) != MK_OK || n_layers < 1) return 0;
  mk::StepPlan sp;  // the row groups run one after another in one workspace
  mk::plan_phases(*layer0, n_layers, mk::group_rows(M, 0), mk::kMaxG, sp);
  return sp.ok ? sp.total : 0;
}


int mk_q4k_step(const mk_q4k_layer* layers, const mk_q4k_layer_io* io, int n_layers, int M,
                const uint16_t* x0, uint16_t* x_out, void* workspace, size_t ws_bytes,
                void* stream) {
  using namespace mk;
  int rc = check_step_shapes(layers, n_layers, M);
  if (rc != MK_OK) return rc;
  if (!io || !x0 || !x_out || !workspace) return MK_EINVAL;
  if (!al16(x0) || !al16(x_out) || !al16(workspace)) return MK_EALIGN;
  for (int l = 0; l < n_layers; ++l) {
    rc = check_layer_io(layers, io[l].y, io[l].x, l);
    if (rc != MK_OK) return rc;
  }
  const bool q6 = any_q6(layers, n_layers);
  // every row group's plan is checked before any work is enqueued (the
  // first group has the most rows)
  StepPlan sp;
  size_t lds = 0;
  int G = 0;
  const int groups = (M + STEP_MAX_M - 1) / STEP_MAX_M;
  for (int g = groups - 1; g >= 0; --g) {
    rc = prepare_walk<0>(layers, n_layers, group_rows(M, g), ws_bytes, q6, sp, lds, G);
    if (rc != MK_OK) return rc;
  }
  const int H = layers[0].q.K;
  std::vector<DevLayer> table(n_layers);
  for (int g = 0; g < groups; ++g) {
    const int r0 = g * STEP_MAX_M, Mg = group_rows(M, g);
    for (int l = 0; l < n_layers; ++l) fill_table(layers[l], io[l].y, io[l].x, r0, table[l]);
    rc = prepare_walk<0>(layers, n_layers, Mg, ws_bytes, q6, sp, lds, G);
    if (rc != MK_OK) return rc;
    rc = enqueue_walk<0>(layers, table, n_layers, Mg, x0 + (size_t)r0 * H, x_out + (size_t)r0 * H,
                         nullptr, workspace, sp, lds, G, g, q6, stream);
    if (rc != MK_OK) return rc;
  }
  return MK_OK;
}

int mk_q4k_step_res(const mk_q4k_layer* layers, const mk_q4k_layer_norm* norms,
                    const mk_q4k_layer_res_io* io, int n_layers, int M, const float* h0,
                    void* workspace, size_t ws_bytes, void* stream) {
  using namespace mk;
  int rc = check_step_shapes(layers, n_layers, M);
  if (rc != MK_OK) return rc;
  if (!io || !norms || !h0 || !workspace) return MK_EINVAL;
  if (!al16(h0) || !al16(workspace)) return MK_EALIGN;
  for (int l = 0; l < n_layers; ++l) {
    rc = check_layer_io(layers, io[l].y, io[l].x, l);
    if (rc != MK_OK) return rc;
    if (!io[l].h_mid || !io[l].h_out || !norms[l].attn || !norms[l].ffn) return MK_EINVAL;
    if (!al16(io[l].h_mid) || !al16(io[l].h_out) || !al16(norms[l].attn) ||
        !al16(norms[l].ffn))
      return MK_EALIGN;
  }
  const bool q6 = any_q6(layers, n_layers);
  StepPlan sp;
  size_t lds = 0;
  int G = 0;
  const int groups = (M + STEP_MAX_M - 1) / STEP_MAX_M;
  for (int g = groups - 1; g >= 0; --g) {
    rc = prepare_walk<1>(layers, n_layers, group_rows(M, g), ws_bytes, q6, sp, lds, G);
    if (rc != MK_OK) return rc;
  }
  const int H = layers[0].q.K;
  std::vector<DevLayer> table(n_layers);
  for (int g = 0; g < groups; ++g) {
    const int r0 = g * STEP_MAX_M, Mg = group_rows(M, g);
    for (int l = 0; l < n_layers; ++l) {
      fill_table(layers[l], io[l].y, io[l].x, r0, table[l]);
      table[l].h[0] = io[l].h_mid + (size_t)r0 * H;
      table[l].h[1] = io[l].h_out + (size_t)r0 * H;
      table[l].g[0] = norms[l].attn;
      table[l].g[1] = norms[l].ffn;
    }
    rc = prepare_walk<1>(layers, n_layers, Mg, ws_bytes, q6, sp, lds, G);
    if (rc != MK_OK) return rc;
    rc = enqueue_walk<1>(layers, table, n_layers, Mg, nullptr, nullptr, h0 + (size_t)r0 * H,
                         workspace, sp, lds, G, g, q6, stream);
    if (rc != MK_OK) return rc;
  }
  return MK_OK;
}

int mk_q4k_step_status(const void* workspace, int* status_out) {
  if (!workspace || !status_out) return MK_EINVAL;
  // the status word sits right after the finished-tile counters
  const size_t off = mk::align256((size_t)mk::DONE_CTRS * mk::CTR_STRIDE * sizeof(unsigned));
  int v = 0;
  if (hipMemcpy(&v, static_cast<const char*>(workspace) + off, sizeof(int),
                hipMemcpyDeviceToHost) != hipSuccess)
    return MK_EHIP;
  *status_out = v;
  return MK_OK;
}

}  // extern "C"
