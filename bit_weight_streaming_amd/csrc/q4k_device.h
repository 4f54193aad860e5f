// q4k_device.h - device building blocks of the Q4_K weight-streaming GEMM
// for gfx950 (CDNA4, wave64, MFMA).
//
// One wave multiplies a "tile" of 16 weight rows (16 output columns n) by up
// to 16*MT stacked activation rows, one 256-weight super-block at a time. The
// weight bytes are streamed from HBM once; the activations sit in LDS.
//
// Per super-block and wave:
//   lane l = n + 16*g (n = l % 16 column of the tile, g = l / 16 in 0..3)
//   loads the 16-byte block header (d, dmin, 12 scale bytes) and the 32 quant
//   bytes of chunk g (quant byte i of chunk g holds weight 64g+i in its low
//   nibble and weight 64g+32+i in its high nibble, i.e. sub-blocks 2g, 2g+1).
//   Nibbles become binary16 operands sc_j * q exactly (sc_j * q <= 945 fits
//   in 11 bits) through the 0x6400 exponent trick and one packed FMA; eight
//   MFMA 16x16x32 f16 instructions contract them with the activations:
//       C_main[m][n] = sum_{k in block} (sc_j(k) * q_k) * x[m][k]
//   and one MFMA 16x16x32 f16 gives the min term
//       C_min[m][n] = sum_j m_j * xsum[m][j]
//   with each fp32 sub-block sum carried as three binary16 parts,
//   xsum = 64 a + b + c (see split_xsum), against (64 m_j, m_j, m_j, 0);
//   then acc[m][n] += d * C_main - dmin * C_min   in fp32.
// This is the factored form of w = d*sc_j*q - dmin*m_j: every product inside
// the MFMA is exact (11-bit * 11-bit significands), so the only roundings are
// fp32 accumulations. Their size follows the two terms, d*sc*q*x and
// dmin*m*x, not their difference w*x: where the two nearly cancel (w close
// to 0 over a whole sub-block) the error is a small multiple of 2^-24 times
// sum(|d sc q x| + |dmin m x|), which can exceed 1e-4 * sum|w x|.
//
// The k order inside one MFMA is free as long as both operands use it; the
// nibble extraction yields pairs (k, k+2) per 32-bit lane-half, so the
// activations are stored in LDS already permuted into that order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mk {

typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef _Float16 half4v __attribute__((ext_vector_type(4)));
typedef _Float16 half8v __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int QK = 256;
constexpr int BLOCK_BYTES = 144;
// LDS bytes per activation row per super-block (256 binary16 values)
constexpr int X_BYTES_PER_BLOCK = 512;
// LDS bytes per activation row per super-block for the sub-block sums
// (8 sub-blocks x {a, b, c, 0} binary16, see split_xsum)
constexpr int XSUM_BYTES_PER_BLOCK = 64;
// Bytes after each row's sub-block sums in LDS: the 16 lanes that read one
// block's sums of 16 rows then hit 16 different bank groups (with a stride of
// a multiple of 128 bytes they would all hit the same one).
constexpr int XSUM_ROW_PAD = 16;
__host__ __device__ constexpr int xsum_row_bytes(int nkb) {
  return nkb * XSUM_BYTES_PER_BLOCK + XSUM_ROW_PAD;
}
// pad added to each LDS activation row so that the 16 rows read by one
// ds_read_b128 land on distinct banks
constexpr int X_ROW_PAD = 16;

template <typename T, typename F>
__device__ __forceinline__ T bit_cast_(F f) {
  static_assert(sizeof(T) == sizeof(F), "size");
  T t;
  __builtin_memcpy(&t, &f, sizeof(T));
  return t;
}

// The three 16-byte loads of one lane for one super-block.
struct BlockRegs {
  u32x4 h;   // d | dmin<<16, scale bytes 0-3, 4-7, 8-11
  u32x4 q0;  // quant bytes 0..15 of chunk g
  u32x4 q1;  // quant bytes 16..31 of chunk g
};

// Streaming loads (nontemporal: each weight byte is used exactly once).
__device__ __forceinline__ void load_block(BlockRegs& r, const uint8_t* blk, int g) {
  r.h = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(blk));
  r.q0 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(blk + 16 + 32 * g));
  r.q1 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(blk + 32 + 32 * g));
}

// binary16 pair (v, v) of a small non-negative integer v <= 63, exactly:
// 0x6400 | v is 1024 + v, minus 1024.
__device__ __forceinline__ half2v small_int_pair(uint32_t v) {
  uint32_t u = (v * 0x00010001u) | 0x64006400u;
  return bit_cast_<half2v>(u) - half2v{(_Float16)1024.0f, (_Float16)1024.0f};
}

// Per-lane constants of the weight unpack and of the scale decode, built once
// per lane (they depend on the lane's group g = lane / 16 only) and kept in
// VGPRs: the nibble masks and exponent patterns of unpack_pair_k, and the
// byte selectors of lane_scales.
struct UnpackConsts {
  uint32_t mlo, mhi;  // low and high nibble of each byte pair
  uint32_t orv, orh;  // binary16 exponent patterns: 1024 + q (low), 64 + q (high)
  uint32_t selA;      // v_perm selector: the scale (min) bytes of sub-blocks 2g, 2g+1
  uint32_t selB;      // v_perm selector: the bytes holding their top 2 bits (g >= 2)
  uint32_t mA;        // mask of the first: 6 bits (g < 2) or the low nibble (g >= 2)
  uint32_t shC;       // shift of the min bytes: 0 (g < 2) or 4 (high nibble, g >= 2)
};

__device__ __forceinline__ UnpackConsts unpack_consts(int g) {
  UnpackConsts k;
  asm volatile("v_mov_b32 %0, 0x000F000F" : "=v"(k.mlo));
  asm volatile("v_mov_b32 %0, 0x00F000F0" : "=v"(k.mhi));
  asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(k.orv));
  asm volatile("v_mov_b32 %0, 0x54005400" : "=v"(k.orh));
  // v_perm bytes: 0-3 pick the second source's bytes, 4-7 the first's, 12
  // gives zero; results hold two values in bytes 0 and 2
  const uint32_t z = 0x0C000C00u;
  if (g < 2) {  // sub-blocks 0..3: 6 bits of scale byte j, min byte j + 4
    k.selA = z | ((uint32_t)(2 * g + 1) << 16) | (uint32_t)(2 * g);
    k.selB = 0x0C0C0C0Cu;  // no top bits
    k.mA = 0x003F003Fu;
    k.shC = 0;
  } else {  // sub-blocks 4..7: nibbles of bytes 8..11, top bits in bytes 0..7
    const uint32_t b0 = 2u * (uint32_t)(g - 2);
    k.selA = z | ((4u + b0 + 1u) << 16) | (4u + b0);
    k.selB = z | ((b0 + 1u) << 16) | b0;
    k.mA = 0x000F000Fu;
    k.shC = 4;
  }
  return k;
}

// Per-lane scale data of one block for sub-blocks 2g (low nibbles) and 2g+1
// (high nibbles).
struct LaneScales {
  half2v sl, nl;  // (sc_lo, sc_lo), (-1024*sc_lo, ...): maps 1024+q -> sc_lo*q
  half2v sh, nh;  // (sc_hi, sc_hi), (-64*sc_hi, ...): maps 64+q -> sc_hi*q
  half8v bmin;    // (64 m_lo, 64 m_hi, m_lo, m_hi, m_lo, m_hi, 0, 0): min-term MFMA operand
  float d, dmin;
};

// The 6-bit scales and mins of sub-blocks 2g, 2g+1 from the block header h
// (h.x: d, dmin; h.y, h.z, h.w: the 12 scale bytes). Sub-blocks 0..3: scale =
// low 6 bits of scale byte j, min = of byte j+4. Sub-blocks 4..7: low 4 bits
// in the low (scale) or high (min) nibble of byte j+4, top 2 bits in bits 6-7
// of byte j-4 (scale) or byte j (min). Each pair is gathered with byte
// permutes into the two halves of a dword, ORed with the exponent of 1024 and
// turned into binary16 (1024 + v) - 1024 = v, exactly.
__device__ __forceinline__ LaneScales lane_scales(const u32x4& h, const UnpackConsts& k) {
  const uint32_t e = 0x64006400u;
  const uint32_t tsc = (__builtin_amdgcn_perm(h.w, h.y, k.selB) >> 2) & 0x00300030u;
  const uint32_t scp = (__builtin_amdgcn_perm(h.w, h.y, k.selA) & k.mA) | tsc | e;
  const uint32_t tmn = (__builtin_amdgcn_perm(h.w, h.z, k.selB) >> 2) & 0x00300030u;
  const uint32_t mnp = ((__builtin_amdgcn_perm(h.w, h.z, k.selA) >> k.shC) & k.mA) | tmn | e;
  const half2v off = {(_Float16)1024.0f, (_Float16)1024.0f};
  const half2v sc = bit_cast_<half2v>(scp) - off;  // (sc_lo, sc_hi)
  const half2v mn = bit_cast_<half2v>(mnp) - off;  // (m_lo, m_hi)
  const half2v nsc = sc * half2v{(_Float16)-1024.0f, (_Float16)-64.0f};
  const half2v mn64 = mn * half2v{(_Float16)64.0f, (_Float16)64.0f};
  LaneScales s;
  s.sl = half2v{sc.x, sc.x};
  s.sh = half2v{sc.y, sc.y};
  s.nl = half2v{nsc.x, nsc.x};
  s.nh = half2v{nsc.y, nsc.y};
  const _Float16 z = (_Float16)0.0f;
  s.bmin = half8v{mn64.x, mn64.y, mn.x, mn.y, mn.x, mn.y, z, z};
  const half2v dd = bit_cast_<half2v>(h.x);
  s.d = (float)dd.x;
  s.dmin = (float)dd.y;
  return s;
}

// Stage activations of super-blocks [kb0, kb0+nkb) of the M rows of X
// ([M][K] binary16, row stride K) into LDS in the MFMA order above (the
// sub-block sums follow from the staged copy: stage_xsum, after a barrier).
// x_lds row m starts at m * row_stride bytes; position of (block b, chunk g,
// MFMA t, element e) is b*512 + g*128 + t*16 + 2*e and holds
// x[m][(kb0+b)*256 + 64g + 32(t&1) + 8(t>>1) + perm(e)], perm = 0,2,1,3,4,6,5,7.
__device__ __forceinline__ void stage_x(const uint16_t* __restrict__ X, int K, int M, int kb0,
                                        int nkb, char* x_lds, int row_stride, int tid,
                                        int nthreads) {
  const int items = M * nkb * 32;
  for (int it = tid; it < items; it += nthreads) {
    const int t = it & 7;
    const int g = (it >> 3) & 3;
    const int rest = it >> 5;
    const int b = rest % nkb;
    const int m = rest / nkb;
    const int k = (kb0 + b) * QK + 64 * g + 32 * (t & 1) + 8 * (t >> 1);
    const u32x4 v = *reinterpret_cast<const u32x4*>(X + (size_t)m * K + k);
    // halves (0,1 | 2,3 | 4,5 | 6,7) -> (0,2 | 1,3 | 4,6 | 5,7)
    u32x4 o;
    o.x = (v.x & 0xFFFFu) | (v.y << 16);
    o.y = (v.x >> 16) | (v.y & 0xFFFF0000u);
    o.z = (v.z & 0xFFFFu) | (v.w << 16);
    o.w = (v.z >> 16) | (v.w & 0xFFFF0000u);
    *reinterpret_cast<u32x4*>(x_lds + (size_t)m * row_stride + b * X_BYTES_PER_BLOCK + g * 128 +
                              t * 16) = o;
  }
}

}  // namespace mk

namespace mk {


}  // namespace mk

namespace mk {

// Bytes of one 16-row tile record of a super-block (see q4k_repack.hip).
constexpr int TILE_REC = 16 * BLOCK_BYTES;

// Lane l's three operands of one tile record: header of row l%16, quant bytes
// [32g, 32g+16) and [32g+16, 32g+32) of that row (g = l/16). The three loads
// of a wave read 256 (broadcast), 1024 and 1024 contiguous bytes.
// Global-address-space views of pointers that come out of LDS tables (which
// the compiler otherwise treats as generic and accesses with flat
// instructions; flat operations also count against the LDS wait counter).
template <class T>
using gptr = __attribute__((address_space(1))) T*;
template <class T>
__device__ __forceinline__ gptr<T> to_global(T* p) {
  return (gptr<T>)p;
}

__device__ __forceinline__ void load_rec(BlockRegs& r, const uint8_t* rec, int lane) {
  const gptr<const u32x4> g = to_global(reinterpret_cast<const u32x4*>(rec));
  r.h = __builtin_nontemporal_load(g + (lane & 15));
  r.q0 = __builtin_nontemporal_load(g + 16 + lane);
  r.q1 = __builtin_nontemporal_load(g + 80 + lane);
}

// B operands of the two MFMAs fed by quant dwords v0, v1 (8 consecutive
// weights of sub-block 2g in the low nibbles, of 2g+1 in the high nibbles),
// k order (0,2,1,3,4,6,5,7): each nibble q becomes the binary16 1024 + q (a
// low nibble, in mantissa bits 0-3 under the exponent of 1024) or 64 + q (a
// high nibble, in bits 4-7 under the exponent of 64, whose last place is
// 1/16) by OR-ing in the exponent pattern, and one packed FMA with (scale,
// -1024 * scale) or (scale, -64 * scale) leaves exactly scale * q: every
// operand and result is exact in binary16. Masks come in registers.
__device__ __forceinline__ void unpack_pair_k(uint32_t v0, uint32_t v1, const LaneScales& s,
                                              const UnpackConsts& k, half8v& b_lo,
                                              half8v& b_hi) {
  const uint32_t t0 = v0 >> 8, t1 = v1 >> 8;
  const half2v l0 = bit_cast_<half2v>((v0 & k.mlo) | k.orv);
  const half2v l1 = bit_cast_<half2v>((t0 & k.mlo) | k.orv);
  const half2v l2 = bit_cast_<half2v>((v1 & k.mlo) | k.orv);
  const half2v l3 = bit_cast_<half2v>((t1 & k.mlo) | k.orv);
  const half2v h0 = bit_cast_<half2v>((v0 & k.mhi) | k.orh);
  const half2v h1 = bit_cast_<half2v>((t0 & k.mhi) | k.orh);
  const half2v h2 = bit_cast_<half2v>((v1 & k.mhi) | k.orh);
  const half2v h3 = bit_cast_<half2v>((t1 & k.mhi) | k.orh);
  const half2v L0 = __builtin_elementwise_fma(l0, s.sl, s.nl);
  const half2v L1 = __builtin_elementwise_fma(l1, s.sl, s.nl);
  const half2v L2 = __builtin_elementwise_fma(l2, s.sl, s.nl);
  const half2v L3 = __builtin_elementwise_fma(l3, s.sl, s.nl);
  const half2v H0 = __builtin_elementwise_fma(h0, s.sh, s.nh);
  const half2v H1 = __builtin_elementwise_fma(h1, s.sh, s.nh);
  const half2v H2 = __builtin_elementwise_fma(h2, s.sh, s.nh);
  const half2v H3 = __builtin_elementwise_fma(h3, s.sh, s.nh);
  b_lo = half8v{L0.x, L0.y, L1.x, L1.y, L2.x, L2.y, L3.x, L3.y};
  b_hi = half8v{H0.x, H0.y, H1.x, H1.y, H2.x, H2.y, H3.x, H3.y};
}

// One 16-row tile of activations (xa: this lane's 128 LDS bytes of the
// block, always valid - rows past M read a real row whose results are never
// stored) against NB weight records of the same super-block; the main term
// runs as one MFMA chain over the block's eight 32-weight groups (in the
// order of the steps u, low then high nibbles), scaled by d once.
template <int NB>
__device__ __forceinline__ void mma_unit(const BlockRegs* r, int g, const char* xa,
                                         const char* xs, const UnpackConsts& k, floatx4* acc) {
  LaneScales s[NB];
  floatx4 c0[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    s[nb] = lane_scales(r[nb].h, k);
    c0[nb] = floatx4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const half8v a_lo = *reinterpret_cast<const half8v*>(xa + 32 * u);
    const half8v a_hi = *reinterpret_cast<const half8v*>(xa + 32 * u + 16);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const uint32_t v0 = u == 0 ? r[nb].q0.x : u == 1 ? r[nb].q0.z : u == 2 ? r[nb].q1.x : r[nb].q1.z;
      const uint32_t v1 = u == 0 ? r[nb].q0.y : u == 1 ? r[nb].q0.w : u == 2 ? r[nb].q1.y : r[nb].q1.w;
      half8v b_lo, b_hi;
      unpack_pair_k(v0, v1, s[nb], k, b_lo, b_hi);
      c0[nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a_lo, b_lo, c0[nb], 0, 0, 0);
      c0[nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a_hi, b_hi, c0[nb], 0, 0, 0);
    }
  }
  const half8v am = *reinterpret_cast<const half8v*>(xs);
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    floatx4 cn = {0.f, 0.f, 0.f, 0.f};
    cn = __builtin_amdgcn_mfma_f32_16x16x32_f16(am, s[nb].bmin, cn, 0, 0, 0);
    const floatx4 dd = {s[nb].d, s[nb].d, s[nb].d, s[nb].d};
    acc[nb] = __builtin_elementwise_fma(dd, c0[nb], acc[nb]);
    acc[nb] = __builtin_elementwise_fma(
        floatx4{-s[nb].dmin, -s[nb].dmin, -s[nb].dmin, -s[nb].dmin}, cn, acc[nb]);
  }
}

}  // namespace mk

namespace mk {

// ---- pieces shared by the persistent streaming kernels (decode step, GEMM)

// Waves per workgroup of the streaming kernels; unit ranges are split over
// them with a shift.
constexpr int SPLIT_WAVES = 8;

// 16-byte device-coherent accesses through a buffer resource (cache policy
// sc1: the agent-scope coherence level, as for relaxed agent-scope atomics).
// Offsets past the resource's size read as zero and drop writes.
constexpr int kCoherent = 16;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}
__device__ __forceinline__ floatx4 ld4_dev(__amdgpu_buffer_rsrc_t r, unsigned off) {
  return __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCoherent));
}
__device__ __forceinline__ void st4_dev(__amdgpu_buffer_rsrc_t r, unsigned off, floatx4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, kCoherent);
}

// Values the compiler cannot see are the same in every lane (read from LDS)
// but are: forcing them into scalar registers keeps the work split and the
// weight-record walk on the scalar unit and out of the vector registers.
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
template <class T>
__device__ __forceinline__ T* uni(T* p) {
  const unsigned long long v = reinterpret_cast<unsigned long long>(p);
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)v);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(v >> 32));
  return reinterpret_cast<T*>(((unsigned long long)hi << 32) | lo);
}

// Work split of one matrix pass over G workgroups: the K range is cut into sk
// slices of nkb super-blocks (the last may be shorter); the workgroups are
// spread over the slices in proportion to their super-blocks, and the nt
// 16-column tiles are split evenly among the workgroups of a slice. Inside a
// workgroup the tw * nkb (tile, super-block) units are split over the waves.
struct Assign {
  int s;      // K slice
  int t0;     // first tile
  int tw;     // tiles
  int kb0;    // first super-block of the slice
  int nkb;    // super-blocks in the slice
  int j, gs;  // index among, and number of, workgroups sharing the slice
  int U;      // units = tw * nkb
};

// First workgroup of slice s.
__host__ __device__ inline int slice_start(int s, int sk, int nkb, int KB, int G) {
  return s >= sk ? G : (int)((long long)G * s * nkb / KB);
}

__host__ __device__ inline Assign assign_split(int nt, int sk, int nkb, int KB, int w, int G) {
  Assign a;
  int s = 0;
  while (s + 1 < sk && slice_start(s + 1, sk, nkb, KB, G) <= w) ++s;
  const int first = slice_start(s, sk, nkb, KB, G);
  a.s = s;
  a.j = w - first;
  a.gs = slice_start(s + 1, sk, nkb, KB, G) - first;
  a.t0 = (int)((long long)nt * a.j / a.gs);
  a.tw = (int)((long long)nt * (a.j + 1) / a.gs) - a.t0;
  a.kb0 = a.s * nkb;
  a.nkb = nkb < KB - a.kb0 ? nkb : KB - a.kb0;
  a.U = a.tw * a.nkb;
  return a;
}

// First unit of wave v's range, and the wave whose range holds unit x (the
// last wave whose range starts at or before x: waves with an empty range are
// skipped). No divisions: both run in the per-tile and per-element loops.
static_assert(SPLIT_WAVES == 8, "wave ranges are computed with a shift by 3");
__host__ __device__ inline int wave_begin(const Assign& a, int v) { return (a.U * v) >> 3; }
__host__ __device__ inline int wave_of_unit(const Assign& a, int x) {
  int w = 0;
#pragma unroll
  for (int v = 1; v < SPLIT_WAVES; ++v) w += ((a.U * v) >> 3) <= x;
  return w;
}

// An fp32 sub-block sum as three binary16 parts, sum = 64 a + b + c: a is
// sum / 64 rounded (|sum| <= 32 * 65504 keeps |a| <= 32752, finite), b the
// rest rounded, c the rest of that. Both subtractions are exact in fp32, so
// the parts hold the sum to about 33 bits where binary16 is normal, and
// exactly whenever it is a multiple of 2^-24 smaller than 2^-3 in magnitude
// (then a = 0 and b, c are exact). The min-term MFMA multiplies them by
// (64 m, m, m): products of 11- and 12-bit significands, exact in fp32.
__device__ __forceinline__ half4v split_xsum(float sum) {
  const _Float16 a = (_Float16)(sum * 0.015625f);
  const float r = sum - 64.f * (float)a;
  const _Float16 b = (_Float16)r;
  const _Float16 c = (_Float16)(r - (float)b);
  return half4v{a, b, c, (_Float16)0.0f};
}

// Store the split_xsum parts (a, b, c) of sub-block j of a block whose 64 LDS
// bytes start at blk: the 16 bytes of the pair 2g, 2g+1 (g = j / 2) hold
// (a_2g, a_2g+1, b_2g, b_2g+1, c_2g, c_2g+1, 0, 0), the order of the min-term
// MFMA operand (see LaneScales::bmin); the even sub-block also writes the
// two zeros.
__device__ __forceinline__ void put_xsum(char* blk, int j, const half4v& p) {
  _Float16* q = reinterpret_cast<_Float16*>(blk + 16 * (j >> 1)) + (j & 1);
  q[0] = p[0];
  q[2] = p[1];
  q[4] = p[2];
  if ((j & 1) == 0) *reinterpret_cast<uint32_t*>(blk + 16 * (j >> 1) + 12) = 0u;
}

// Sub-block sums of the staged activations, as split_xsum parts, for the
// min-term MFMA: row m, block b at xs_lds + m * xs_row + b * 64, in put_xsum's
// order (xs_row = xsum_row_bytes(nkb)).
__device__ __forceinline__ void stage_xsum(int M, int nkb, int xs_row, const char* x_lds,
                                           int x_stride, char* xs_lds, int tid,
                                           int nthreads) {
  // eight neighbouring lanes take eight rows of one (block, sub-block): their
  // reads (row stride = 16 bytes modulo 128) fall on distinct banks
  const int M8 = (M + 7) & ~7;
  const int items = M8 * nkb * 8;
  for (int it = tid; it < items; it += nthreads) {
    const int j = (it >> 3) & 7;
    const int rest = it >> 6;
    const int b = rest % nkb;
    const int m = (rest / nkb) * 8 + (it & 7);
    if (m >= M) continue;
    const int gq = j >> 1, hb = j & 1;
    float sum = 0.f;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(
          x_lds + (size_t)m * x_stride + b * X_BYTES_PER_BLOCK + gq * 128 + (2 * u + hb) * 16);
      const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const half2v hh = bit_cast_<half2v>(w4[i]);
        sum += (float)hh.x;
        sum += (float)hh.y;
      }
    }
    put_xsum(xs_lds + (size_t)m * xs_row + b * XSUM_BYTES_PER_BLOCK, j, split_xsum(sum));
  }
}

// Activations of MT 16-row tiles (xa[rt]: this lane's 128 LDS bytes of the
// block, always valid - rows past M read a real row whose results are never
// stored) against one weight record; the main term runs as one MFMA chain per
// row tile (as mma_unit), the weights are unpacked once for all row tiles.
template <int MT>
__device__ __forceinline__ void mma_unit_mt(const BlockRegs& r, int g, const char* const* xa,
                                            const char* const* xs, const UnpackConsts& k,
                                            floatx4* acc) {
  const LaneScales s = lane_scales(r.h, k);
  floatx4 c0[MT];
#pragma unroll
  for (int rt = 0; rt < MT; ++rt) c0[rt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const uint32_t v0 = u == 0 ? r.q0.x : u == 1 ? r.q0.z : u == 2 ? r.q1.x : r.q1.z;
    const uint32_t v1 = u == 0 ? r.q0.y : u == 1 ? r.q0.w : u == 2 ? r.q1.y : r.q1.w;
    half8v b_lo, b_hi;
    unpack_pair_k(v0, v1, s, k, b_lo, b_hi);
#pragma unroll
    for (int rt = 0; rt < MT; ++rt) {
      const half8v a_lo = *reinterpret_cast<const half8v*>(xa[rt] + 32 * u);
      const half8v a_hi = *reinterpret_cast<const half8v*>(xa[rt] + 32 * u + 16);
      c0[rt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a_lo, b_lo, c0[rt], 0, 0, 0);
      c0[rt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a_hi, b_hi, c0[rt], 0, 0, 0);
    }
  }
  const floatx4 dd = {s.d, s.d, s.d, s.d};
  const floatx4 nm = {-s.dmin, -s.dmin, -s.dmin, -s.dmin};
#pragma unroll
  for (int rt = 0; rt < MT; ++rt) {
    const half8v am = *reinterpret_cast<const half8v*>(xs[rt]);
    floatx4 cn = {0.f, 0.f, 0.f, 0.f};
    cn = __builtin_amdgcn_mfma_f32_16x16x32_f16(am, s.bmin, cn, 0, 0, 0);
    acc[rt] = __builtin_elementwise_fma(dd, c0[rt], acc[rt]);
    acc[rt] = __builtin_elementwise_fma(nm, cn, acc[rt]);
  }
}

}  // namespace mk

namespace mk {

// ---- Q6_K matrices inside the decode-step walk
//
// Q6_K (the other k-quant a Q4_K_M file holds, for attn_v and ffn_down):
// 256 weights in 210 bytes per row and block, ql[128] low nibbles, qh[64]
// high bit pairs, 16 int8 run scales, binary16 d; weight k (half h = k/128,
// quarter j = (k % 128) / 32, place l = k % 32) has low bits nibble j/2 of
// ql[64h + 32 (j % 2) + l], high bits 2j..2j+1 of qh[32h + l], q = low |
// high << 4 and value d * sc[k / 16] * (q - 32).
//
// The walk stages its activations once per phase in the MFMA order of the
// Q4_K product (16x16x32: lane l = 16 g + c takes row c and the 64 weights
// [64g, 64g+64) of each block), so a Q6_K matrix in the walk is repacked at
// load time (mk_q6k_step_repack) into records of 16 rows x one block in that
// same lane order, 3360 bytes (16 x 210, nothing added):
//   [0, 1024)     lane l: bytes i = 0..15: low nibble = low bits of weight
//                 64g + i, high nibble = of weight 64g + 32 + i
//   [1024, 2048)  lane l: the same for weights 64g + 16 + i, 64g + 48 + i
//   [2048, 3072)  lane l: high bit pairs, 16 bytes: byte 4m + b holds, in
//                 bits 0-1, 2-3, 4-5 and 6-7, those of weights 64g + 8m + b,
//                 64g + 32 + 8m + b, 64g + 8m + 4 + b, 64g + 36 + 8m + b
//   [3072, 3328)  lane l: the int8 scales of runs 4g .. 4g+3 of row c
//   [3328, 3360)  row c's d at 3328 + 2c
// followed, after all records, by the column sums like the Q4_K records.
constexpr int Q6W_REC = 3360;

// A lane's operands of one Q6_K walk record: the quant and high-bit dwords
// in the registers of a Q4_K ring slot (BlockRegs: h = low bits of quant
// dwords 0-3, q0 = of 4-7, q1 = high bit pairs, dword m for quant dwords 2m
// and 2m+1), so that a walk's Q6_K records stream through the same ring;
// plus the lane's run scales and its row's d.
struct ScaleRegs6 {
  uint32_t sc;  // int8 scales of runs 4g .. 4g+3
  uint32_t d;   // binary16 d of the lane's row (low half)
};

__device__ __forceinline__ void load_rec6(BlockRegs& r, ScaleRegs6& s, const uint8_t* rec,
                                          int lane) {
  typedef __attribute__((address_space(1))) const u32x4 g4;
  typedef __attribute__((address_space(1))) const uint32_t g1;
  typedef __attribute__((address_space(1))) const uint16_t gh;
  const auto g = to_global(rec);
  r.h = __builtin_nontemporal_load(reinterpret_cast<g4*>(g) + lane);
  r.q0 = __builtin_nontemporal_load(reinterpret_cast<g4*>(g + 1024) + lane);
  r.q1 = __builtin_nontemporal_load(reinterpret_cast<g4*>(g + 2048) + lane);
  s.sc = __builtin_nontemporal_load(reinterpret_cast<g1*>(g + 3072) + lane);
  s.d = __builtin_nontemporal_load(reinterpret_cast<gh*>(g + 3328) + (lane & 15));
}

// binary16 (1024 + q) of the bytes (0, 2) and (1, 3) of a dword of 6-bit codes,
// as two pairs: the MFMA element order 0, 2, 1, 3 within four weights.
__device__ __forceinline__ void q6_codes_f16(uint32_t q, uint32_t& p02, uint32_t& p13) {
  p02 = __builtin_amdgcn_perm(0x64646464u, q, 0x04020400u);
  p13 = __builtin_amdgcn_perm(0x64646464u, q, 0x04030401u);
}

// B operands (hi and lo parts) of one 16x16x32 MFMA from the 8 weights of
// quant dwords ve, vo with their high bits already in bits 4-5 of each byte
// (codes qe, qo): s * (q - 32) for scale pair s, split as hi = fl(s * t)
// plus lo = s * t - hi (exact with one fused multiply-add: the integers
// s * t <= 4096 in magnitude leave a rounding error of at most 1), so the two
// MFMAs together multiply by the exact scaled weight.
__device__ __forceinline__ void q6_operands(uint32_t qe, uint32_t qo, half2v s, half8v& hi,
                                            half8v& lo) {
  uint32_t f[4];
  q6_codes_f16(qe, f[0], f[1]);
  q6_codes_f16(qo, f[2], f[3]);
  const half2v off = {(_Float16)1056.0f, (_Float16)1056.0f};
  half2v h[4], l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const half2v t = bit_cast_<half2v>(f[i]) - off;  // q - 32, exact
    h[i] = t * s;
    l[i] = __builtin_elementwise_fma(t, s, -h[i]);
  }
  hi = half8v{h[0].x, h[0].y, h[1].x, h[1].y, h[2].x, h[2].y, h[3].x, h[3].y};
  lo = half8v{l[0].x, l[0].y, l[1].x, l[1].y, l[2].x, l[2].y, l[3].x, l[3].y};
}

// MT 16-row tiles of staged activations (xa[rt]: this lane's 128 LDS bytes of
// the block in tile rt, as for Q4_K) against one Q6_K walk record: for each
// step u the lower MFMA takes weights 64g + 8u + (0..7) (run 4g + u/2), the
// upper 64g + 32 + 8u + (0..7) (run 4g + 2 + u/2); the weight operands are
// built once for all tiles; acc[rt] += d * (sum of both chains).
template <int MT>
__device__ __forceinline__ void mma_unit6_mt(const BlockRegs& r, const ScaleRegs6& rs,
                                             const char* const* xa, floatx4* acc) {
  half2v sc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const _Float16 v = (_Float16)(float)(int)(int8_t)(rs.sc >> (8 * i));
    sc[i] = half2v{v, v};
  }
  floatx4 c0[MT], c1[MT];
#pragma unroll
  for (int rt = 0; rt < MT; ++rt) c0[rt] = c1[rt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const uint32_t ve = u == 0 ? r.h.x : u == 1 ? r.h.z : u == 2 ? r.q0.x : r.q0.z;
    const uint32_t vo = u == 0 ? r.h.y : u == 1 ? r.h.w : u == 2 ? r.q0.y : r.q0.w;
    const uint32_t H = u == 0 ? r.q1.x : u == 1 ? r.q1.y : u == 2 ? r.q1.z : r.q1.w;
    const uint32_t m4 = 0x0F0F0F0Fu, m2 = 0x30303030u;
    const uint32_t qle = (ve & m4) | ((H << 4) & m2), qlo = (vo & m4) | (H & m2);
    const uint32_t qhe = ((ve >> 4) & m4) | ((H << 2) & m2), qho = ((vo >> 4) & m4) | ((H >> 2) & m2);
    half8v bh, bl;
    q6_operands(qle, qlo, sc[u >> 1], bh, bl);
#pragma unroll
    for (int rt = 0; rt < MT; ++rt) {
      const half8v a_lo = *reinterpret_cast<const half8v*>(xa[rt] + 32 * u);
      c0[rt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a_lo, bh, c0[rt], 0, 0, 0);
      c0[rt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a_lo, bl, c0[rt], 0, 0, 0);
    }
    q6_operands(qhe, qho, sc[2 + (u >> 1)], bh, bl);
#pragma unroll
    for (int rt = 0; rt < MT; ++rt) {
      const half8v a_hi = *reinterpret_cast<const half8v*>(xa[rt] + 32 * u + 16);
      c1[rt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a_hi, bh, c1[rt], 0, 0, 0);
      c1[rt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a_hi, bl, c1[rt], 0, 0, 0);
    }
  }
  const float d = (float)bit_cast_<_Float16>((uint16_t)rs.d);
  const floatx4 dd = {d, d, d, d};
#pragma unroll
  for (int rt = 0; rt < MT; ++rt) {
    acc[rt] = __builtin_elementwise_fma(dd, c0[rt], acc[rt]);
    acc[rt] = __builtin_elementwise_fma(dd, c1[rt], acc[rt]);
  }
}

// The walk's case: one row tile.
__device__ __forceinline__ void mma_unit6(const BlockRegs& r, const ScaleRegs6& rs,
                                          const char* xa, floatx4& acc) {
  const char* xas[1] = {xa};
  mma_unit6_mt<1>(r, rs, xas, &acc);
}

}  // namespace mk
