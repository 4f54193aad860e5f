// q8_attn.hip - decode attention of stacked rows over a paged q8_0 KV pool.
//
// The decode step's other growing cost (the OpenJet post, "RTX 3090 one
// card, four coding agents", paragraph on how parallel decoding works: with
// the weights read once per step, what grows with the agents is attention
// over their caches). Each agent's R rows (next token + drafts) attend to
// the agent's cached tokens, held in 16-token pages of a shared pool and
// listed in a per-agent page table; row j sees the agent's first row_len
// tokens. Heads are grouped over KV heads (n_heads / n_kv query heads each).
//
// Work split: one workgroup of 4 waves per (agent, KV head, group of
// 4 * ppw pages); wave w takes ppw consecutive pages of the group (ppw = 16
// for page tables of 2048 pages and more, fewer for narrower tables). All R x group
// query vectors of the (agent, KV head) ride in one wave (up to 32: two
// 16-column MFMA tiles), so every K and V byte is read once per step.
//
// Per page (16 tokens), with MFMA (binary16 scores, bfloat16 values, fp32
// accumulate):
//   scores  S^T[t][q] = sum_u ks[t][u] * (Kq_u . Q_u)  - four 16x16x32 MFMAs
//           per query tile, one per 32-dim q8_0 block u, the int8 quants
//           entering exactly and each block's scale applied to its product;
//   softmax online over the pages, in the log2 domain, per query column;
//   values  O^T[d][q] += sigma * (Vq^T . B), B[t][q] = p[t][q] * vs[t][b] /
//           sigma * 2^12 split exactly into three bfloat16 parts (three
//           16x16x16 MFMAs per 16-dim tile, the quants as bfloat16), sigma a
//           power of two at least the page's largest V scale, so B is at
//           most 2^12; the 2^12 is taken out at the end.
// S^T comes out of the score MFMA in exactly the register layout the value
// MFMA wants for its B operand (4 consecutive tokens of one query per lane),
// so no transpose is needed.
// The 4 waves' states merge in LDS; each workgroup writes one partial
// (running max, sum, 128 outputs per query vector) and q8_attn_merge adds the
// partials of each (row, head) in group order. Everything is deterministic.
#include <math.h>
#include <string.h>

#include "mk_q4k.h"
#include "mk_q8attn.h"
#include "q4k_device.h"

namespace mk {

namespace {

constexpr int ATT_WAVES = 4;
constexpr int ATT_THREADS = 64 * ATT_WAVES;
constexpr int PAGE_TOKENS = 16;
constexpr int HEAD_DIM = 128;
constexpr int PAGE_HEAD_BYTES = 4352;
constexpr int MAX_PAGES_PER_WAVE = 16;

// Pages per wave for a page table max_pages wide: 16 from 2048 pages (32k
// tokens) up, halving below, at least 2, so that short caches still spread
// over the chip. It depends on the table width only, never on the actual
// lengths or the number of agents, so a row's summation order does not
// depend on the other rows of the call.
__host__ __device__ inline int pages_per_wave(int max_pages) {
  int ppw = MAX_PAGES_PER_WAVE;
  while (ppw > 2 && max_pages < 128 * ppw) ppw >>= 1;
  return ppw;
}
constexpr int TILES_PER_WAVE = 8 / ATT_WAVES;  // output tiles each wave merges
constexpr int MAX_QV = 32;        // query vectors per (agent, KV head)
constexpr int PART_FLOATS = 132;  // per query vector: max, sum, 128 outputs, pad
constexpr float P_SCALE = 4096.f;  // 2^12


struct AttnArgs {
  const uint16_t* q;        // [M][n_heads][128] binary16
  const uint8_t* pool;      // pages
  const int32_t* table;     // [n_agents][max_pages]
  const int32_t* row_len;   // [M]
  float* part;              // [n_agents][n_kv][max_groups][MAX_QV][PART_FLOATS]
  float* out;               // [M][n_heads][128]
  int n_agents, rows, max_pages, n_heads, n_kv, group, nqv, max_groups, n_pages;
  int ppw;                  // pages per wave; a workgroup's group is 4 * ppw pages
  float qk_scale;           // log2(e) / sqrt(128)
};

__device__ __forceinline__ float xor_max(float v, int m) {
  return fmaxf(v, __shfl_xor(v, m, 64));
}
__device__ __forceinline__ float xor_sum(float v, int m) { return v + __shfl_xor(v, m, 64); }

// The max over lanes c, c + 16, c + 32, c + 48 (the four rows of a 16-lane
// column) in every one of them, with the gfx950 row swaps (VALU, no LDS
// round trip): swapping two copies of v between odd and even rows, then
// between the wave's halves, leaves each pair holding complementary rows.
// (Both outputs of a swap pass through an empty asm: fed one value twice,
// the compiler may otherwise take them for equal and drop the max.)
template <bool ROWS16>
__device__ __forceinline__ void swap_pair(uint32_t v, uint32_t& x, uint32_t& y) {
  const auto a = ROWS16 ? __builtin_amdgcn_permlane16_swap(v, v, false, false)
                        : __builtin_amdgcn_permlane32_swap(v, v, false, false);
  x = a[0];
  y = a[1];
  asm volatile("" : "+v"(x), "+v"(y));
}
__device__ __forceinline__ uint32_t col_max_u32(uint32_t v) {
  uint32_t x, y;
  swap_pair<true>(v, x, y);
  swap_pair<false>(max(x, y), x, y);
  return max(x, y);
}
__device__ __forceinline__ float col_max(float v) {
  uint32_t x, y;
  swap_pair<true>(__builtin_bit_cast(uint32_t, v), x, y);
  v = fmaxf(__builtin_bit_cast(float, x), __builtin_bit_cast(float, y));
  swap_pair<false>(__builtin_bit_cast(uint32_t, v), x, y);
  return fmaxf(__builtin_bit_cast(float, x), __builtin_bit_cast(float, y));
}

// Tokens row r attends to, clamped to what the page table can list.
__device__ __forceinline__ int row_tokens(const AttnArgs& A, int r) {
  return min(max(A.row_len[r], 0), A.max_pages * PAGE_TOKENS);
}

// Tokens agent a's rows attend to at most.
__device__ __forceinline__ int agent_len(const AttnArgs& A, int a) {
  int n = 0;
  for (int j = 0; j < A.rows; ++j) n = max(n, row_tokens(A, a * A.rows + j));
  return n;
}

// One page-head's bytes as lane l = 16 g + c holds them: K quants of token
// c, dims 32u + 8g .. +7 (u = 0..3); K scales of tokens 4g .. 4g+3 (4 blocks
// each); V quants of dims 16 dt + c, tokens 4g .. 4g+3 (dt = 0..7); V scales
// of tokens 4g .. 4g+3. The pool layout puts the quants in four 1 KiB slabs
// whose 16 bytes at 16 l are exactly lane l's (slab 0: u = 0, 1; slab 1:
// u = 2, 3; slab 2: dt = 0..3; slab 3: dt = 4..7), and the scales of the
// lane's four tokens in the 64 bytes at 4096 + 64 g (K then V).
struct PageRaw {
  u32x4 q[4];
  u32x4 ks[2];
  u32x4 vs[2];
};

__device__ __forceinline__ void load_page(PageRaw& R, const uint8_t* ph, int c, int g) {
  const int l = 16 * g + c;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    R.q[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(ph + 1024 * i + 16 * l));
  const u32x4* sc = reinterpret_cast<const u32x4*>(ph + 4096 + 64 * g);  // shared by 16 lanes
  R.ks[0] = sc[0];
  R.ks[1] = sc[1];
  R.vs[0] = sc[2];
  R.vs[1] = sc[3];
}

// binary16 number i (0..15) of a 32-byte scale group
__device__ __forceinline__ float half_at(const u32x4 (&w)[2], int i) {
  const uint32_t x = w[i >> 3][(i >> 1) & 3];
  return (float)bit_cast_<_Float16>((uint16_t)(x >> (16 * (i & 1))));
}

// 2^k for the exponent field k of a normal float: exact, no division
__device__ __forceinline__ float pow2_field(int k) { return __builtin_bit_cast(float, (uint32_t)k << 23); }

// Four int8 numbers (a little-endian word) as exact binary16: each byte,
// offset by 128, becomes the low mantissa byte of 1024 (binary16 0x6400), and
// 1152 = 1024 + 128 is then subtracted in binary16, exactly.
__device__ __forceinline__ half4v i8x4_to_h4(uint32_t w) {
  const uint32_t u = w ^ 0x80808080u;
  const u32x2 b = {__builtin_amdgcn_perm(0x64646464u, u, 0x04010400u),
                   __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u)};
  const _Float16 k = (_Float16)1152.f;
  return __builtin_bit_cast(half4v, b) - half4v{k, k, k, k};
}

// The value weights enter the matrix cores as three bfloat16 parts, which
// add up to the fp32 weight exactly: hi = w truncated to bfloat16 (its top
// 16 bits), r = w - hi (exact in fp32: the low 16 bits of w's significand),
// mid = r truncated, lo = r - mid (exact, and at most 8 significant bits, so
// it is a bfloat16 as it stands). bfloat16 keeps fp32's exponent range, so
// the split holds every weight, however small, down to fp32's normal range,
// with no rebasing. The value quants enter as bfloat16 too: an int8 is exact.
typedef short bf16x4 __attribute__((ext_vector_type(4)));

// bfloat16 pair {a, b} (a in the low half) of two fp32 numbers whose low 16
// bits are to be dropped
__device__ __forceinline__ uint32_t bf_pair(float a, float b) {
  return __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, b), __builtin_bit_cast(uint32_t, a),
                               0x07060302u);
}
__device__ __forceinline__ float bf_trunc(float v) {
  return __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, v) & 0xFFFF0000u);
}
__device__ __forceinline__ void split3(float v0, float v1, uint32_t& hi, uint32_t& mid,
                                       uint32_t& lo) {
  hi = bf_pair(v0, v1);
  const float r0 = v0 - bf_trunc(v0), r1 = v1 - bf_trunc(v1);
  mid = bf_pair(r0, r1);
  lo = bf_pair(r0 - bf_trunc(r0), r1 - bf_trunc(r1));
}

// Four int8 numbers (a little-endian word) as exact bfloat16: each converted
// to fp32 (at most 8 significant bits, so the top 16 bits hold it).
__device__ __forceinline__ bf16x4 i8x4_to_bf4(uint32_t w) {
  const float f0 = (float)(int)(int8_t)(w & 0xFFu), f1 = (float)(int)(int8_t)((w >> 8) & 0xFFu);
  const float f2 = (float)(int)(int8_t)((w >> 16) & 0xFFu), f3 = (float)(int)(int8_t)(w >> 24);
  return __builtin_bit_cast(bf16x4, u32x2{bf_pair(f0, f1), bf_pair(f2, f3)});
}

// O^T += V^T * B for one page: B = the page's value weights pv (already
// times 2^12 / sigma) times each token's V scale of block b, as split3's
// three bfloat16 parts, each against the same bfloat16 value quants.
template <int NQT>
__device__ __forceinline__ void value_blocks(const PageRaw& R, const float (&pv)[NQT][4],
                                             floatx4 (&acc)[NQT][8]) {
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    float vsb[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) vsb[r] = half_at(R.vs, 4 * r + b);
    bf16x4 bh[NQT], bm[NQT], bl[NQT];
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt) {
      uint32_t h0, h1, m0, m1, l0, l1;
      float wv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) wv[r] = pv[qt][r] * vsb[r];
      split3(wv[0], wv[1], h0, m0, l0);
      split3(wv[2], wv[3], h1, m1, l1);
      bh[qt] = __builtin_bit_cast(bf16x4, u32x2{h0, h1});
      bm[qt] = __builtin_bit_cast(bf16x4, u32x2{m0, m1});
      bl[qt] = __builtin_bit_cast(bf16x4, u32x2{l0, l1});
    }
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int dt = 2 * b + e;
      const bf16x4 av = i8x4_to_bf4(R.q[2 + (dt >> 2)][dt & 3]);
#pragma unroll
      for (int qt = 0; qt < NQT; ++qt) {
        acc[qt][dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, bh[qt], acc[qt][dt], 0, 0, 0);
        acc[qt][dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, bm[qt], acc[qt][dt], 0, 0, 0);
        acc[qt][dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, bl[qt], acc[qt][dt], 0, 0, 0);
      }
    }
  }
}

template <int NQT>
__global__ void __launch_bounds__(ATT_THREADS, 2) q8_attn_kernel(AttnArgs A) {
  __shared__ floatx4 acc_s[ATT_WAVES][8][64];    // one query tile of every wave
  __shared__ float st_s[ATT_WAVES][NQT][64][2];  // per wave and tile: (max, sum) per lane
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
  const int c = lane & 15, g = lane >> 4;
  const int grp = blockIdx.x % A.max_groups;
  const int kvh = (blockIdx.x / A.max_groups) % A.n_kv;
  const int a = blockIdx.x / (A.max_groups * A.n_kv);
  const int len_a = agent_len(A, a);
  const int npages = (len_a + PAGE_TOKENS - 1) / PAGE_TOKENS;
  const int gpages = ATT_WAVES * A.ppw;
  if (grp * gpages >= npages) return;  // nothing here (uniform per workgroup)
  const int p0 = grp * gpages + wave * A.ppw;
  const int p1 = min(p0 + A.ppw, npages);

  // query operands (B of the score MFMA): query vector 16 qt + c, dims
  // 32 u + 8 g .. +7; columns past the agent's query vectors hold zeros and
  // are never written out
  half8v qop[NQT][4];
  int qlen[NQT];
  int lmin = 0x7FFFFFFF;
#pragma unroll
  for (int qt = 0; qt < NQT; ++qt) {
    const int qv = 16 * qt + c;
    const bool live = qv < A.nqv;
    const int j = live ? qv / A.group : 0, hh = live ? qv % A.group : 0;
    const int row = a * A.rows + j, head = kvh * A.group + hh;
    qlen[qt] = live ? row_tokens(A, row) : 0x7FFFFFFF;
    lmin = min(lmin, qlen[qt]);
    const uint16_t* qp = A.q + ((size_t)row * A.n_heads + head) * HEAD_DIM;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      u32x4 v = live ? *reinterpret_cast<const u32x4*>(qp + 32 * u + 8 * g) : u32x4{0u, 0u, 0u, 0u};
      qop[qt][u] = __builtin_bit_cast(half8v, v);
    }
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) lmin = min(lmin, __shfl_xor(lmin, o, 64));
  // the wave's page list, one entry per lane, clamped into the pool
  const int32_t* tab = A.table + (size_t)a * A.max_pages;
  int pg_l = 0;
  if (lane < A.ppw && p0 + lane < p1) pg_l = min(max(tab[p0 + lane], 0), A.n_pages - 1);
  auto page_ptr = [&](int p) {
    const int pg = __builtin_amdgcn_readlane(pg_l, p - p0);
    return A.pool + ((size_t)pg * A.n_kv + kvh) * PAGE_HEAD_BYTES;
  };

  // running state: per query column the max (raw score units) and this
  // lane's share of the sum; the outputs in units of 2^12 / sigma_run,
  // sigma_run the largest page bound so far
  float m[NQT], lsum[NQT];
  floatx4 acc[NQT][8];
  int ke_run = 0;  // exponent field of sigma_run; 0 before any nonzero V scale
#pragma unroll
  for (int qt = 0; qt < NQT; ++qt) {
    m[qt] = -INFINITY;
    lsum[qt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) acc[qt][dt] = floatx4{0.f, 0.f, 0.f, 0.f};
  }

  auto page_step = [&](const PageRaw& R, int p) {
    const int tok0 = p * PAGE_TOKENS + 4 * g;  // this lane's first token
    const bool full = (p + 1) * PAGE_TOKENS <= lmin;
    float pv[NQT][4], alpha[NQT];
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt)
#pragma unroll
      for (int r = 0; r < 4; ++r) pv[qt][r] = 0.f;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const half4v x = i8x4_to_h4(R.q[u >> 1][2 * (u & 1)]), y = i8x4_to_h4(R.q[u >> 1][2 * (u & 1) + 1]);
      const half8v ka = {x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
#pragma unroll
      for (int qt = 0; qt < NQT; ++qt) {
        const floatx4 su =
            __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, qop[qt][u], floatx4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) pv[qt][r] = __builtin_fmaf(half_at(R.ks, 4 * r + u), su[r], pv[qt][r]);
      }
    }
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt) {
      // scores stay in raw units (the running max too); the weights are
      // 2^(qk_scale (s - m)), qk_scale = log2(e) / sqrt(128) > 0
      float mp = -INFINITY;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        pv[qt][r] = full || tok0 + r < qlen[qt] ? pv[qt][r] : -INFINITY;
        mp = fmaxf(mp, pv[qt][r]);
      }
      mp = col_max(mp);
      const float mn = fmaxf(m[qt], mp);
      const float ms = mn == -INFINITY ? 0.f : -mn * A.qk_scale;
      alpha[qt] = __builtin_amdgcn_exp2f(__builtin_fmaf(m[qt], A.qk_scale, ms));
      float ps = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        pv[qt][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(pv[qt][r], A.qk_scale, ms));
        ps += pv[qt][r];
      }
      lsum[qt] = __builtin_fmaf(lsum[qt], alpha[qt], ps);
      m[qt] = mn;
    }
    // the page's V bound: a power of two >= every |scale| of its 16 tokens
    // (on the binary16 bits: |x| orders as its magnitude bits)
    uint32_t vbits = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t w = R.vs[i >> 2][i & 3] & 0x7FFF7FFFu;
      vbits = max(vbits, max(w & 0xFFFFu, w >> 16));
    }
    vbits = col_max_u32(vbits);
    const float vmax = (float)bit_cast_<_Float16>((uint16_t)vbits);
    // sigma as an exponent field (0: no nonzero scale yet); vmax is a
    // binary16 value, so 2^-24 <= sigma <= 2^16 and every power below is normal
    const uint32_t vb = __builtin_bit_cast(uint32_t, vmax);
    const int ke_p = vmax > 0.f ? (int)(((vb + 0x007FFFFFu) & 0xFF800000u) >> 23) : 0;
    const int ke_new = max(ke_run, ke_p);
    const bool grew = ke_new != ke_run;
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt) {
      if (grew || __builtin_amdgcn_ballot_w64(alpha[qt] != 1.f) != 0) {  // uniform branch
        const float f = ke_run > 0 ? alpha[qt] * pow2_field(127 + ke_run - ke_new) : 0.f;
        const floatx4 ff = {f, f, f, f};
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) acc[qt][dt] *= ff;
      }
    }
    ke_run = ke_new;
    // the weights times 2^12 / sigma_run
    const float bscale = ke_run > 0 ? pow2_field(266 - ke_run) : 0.f;
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt)
#pragma unroll
      for (int r = 0; r < 4; ++r) pv[qt][r] *= bscale;
    value_blocks<NQT>(R, pv, acc);
  };

  // two page buffers in registers: the next page's loads are in flight while
  // this one is computed. The loads are unconditional (past the wave's last
  // page they read that page again, just read and still in cache) so that
  // each wait covers exactly the older buffer.
  if (p0 < p1) {
    PageRaw R0, R1;
    load_page(R0, page_ptr(p0), c, g);
    for (int p = p0; p < p1; p += 2) {
      load_page(R1, page_ptr(min(p + 1, p1 - 1)), c, g);
      __builtin_amdgcn_sched_barrier(0);  // the loads go out before the compute
      page_step(R0, p);
      load_page(R0, page_ptr(min(p + 2, p1 - 1)), c, g);
      __builtin_amdgcn_sched_barrier(0);
      if (p + 1 < p1) page_step(R1, p + 1);
    }
  }

  // merge the four waves in LDS (fixed order), one query tile at a time,
  // then one partial per workgroup: (max, sum, 128 outputs x 2^12)
#pragma unroll
  for (int qt = 0; qt < NQT; ++qt) {
    st_s[wave][qt][lane][0] = m[qt] * A.qk_scale;  // log2 units, as the partials
    st_s[wave][qt][lane][1] = xor_sum(xor_sum(lsum[qt], 16), 32);
  }
#pragma unroll
  for (int qt = 0; qt < NQT; ++qt) {
    const float sr = ke_run > 0 ? pow2_field(ke_run) : 0.f;
    const floatx4 sg = {sr, sr, sr, sr};
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) acc_s[wave][dt][lane] = acc[qt][dt] * sg;
    __syncthreads();
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < ATT_WAVES; ++w) mx = fmaxf(mx, st_s[w][qt][lane][0]);
    float L = 0.f;
    floatx4 o[TILES_PER_WAVE];
#pragma unroll
    for (int i = 0; i < TILES_PER_WAVE; ++i) o[i] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < ATT_WAVES; ++w) {
      const float f = mx == -INFINITY ? 0.f : exp2f(st_s[w][qt][lane][0] - mx);
      L = __builtin_fmaf(st_s[w][qt][lane][1], f, L);
      const floatx4 ff = {f, f, f, f};
#pragma unroll
      for (int i = 0; i < TILES_PER_WAVE; ++i)
        o[i] = __builtin_elementwise_fma(ff, acc_s[w][TILES_PER_WAVE * wave + i][lane], o[i]);
    }
    const int qv = 16 * qt + c;
    if (qv < A.nqv) {
      float* dst =
          A.part + ((((size_t)a * A.n_kv + kvh) * A.max_groups + grp) * MAX_QV + qv) * PART_FLOATS;
      if (wave == 0 && g == 0) {
        dst[0] = mx;
        dst[1] = L;
      }
      // tile dt holds dims 16 dt + 4 g .. +3 of query qv
#pragma unroll
      for (int i = 0; i < TILES_PER_WAVE; ++i)
        *reinterpret_cast<floatx4*>(dst + 4 + 16 * (TILES_PER_WAVE * wave + i) + 4 * g) = o[i];
    }
    __syncthreads();
  }
}

constexpr int MERGE_PARTS = 4;
constexpr int MERGE_THREADS = MERGE_PARTS * HEAD_DIM;
constexpr int MERGE_CHUNK = MERGE_THREADS;

// One block per (row, head): add the partials of the row's agent and KV head.
// Thread (part, d) sums output dim d over groups part, part + 4, ... of each
// chunk of 512 groups, the four parts then adding up in fixed order; the
// group weights exp2(max_g - max) go through LDS a chunk at a time. The
// order depends only on the agent's group count.
__global__ void __launch_bounds__(MERGE_THREADS) q8_attn_merge(AttnArgs A) {
  __shared__ float red[MERGE_THREADS / 64];
  __shared__ float fw[MERGE_CHUNK];
  __shared__ float osum[MERGE_PARTS][HEAD_DIM];
  const int tid = threadIdx.x, d = tid % HEAD_DIM, part = tid / HEAD_DIM;
  const int r = blockIdx.x / A.n_heads, h = blockIdx.x % A.n_heads;
  const int a = r / A.rows, j = r % A.rows;
  const int kvh = h / A.group, qv = j * A.group + h % A.group;
  const int npages = (agent_len(A, a) + PAGE_TOKENS - 1) / PAGE_TOKENS;
  const int gpages = ATT_WAVES * A.ppw;
  const int ng = (npages + gpages - 1) / gpages;
  const float* src = A.part + (((size_t)a * A.n_kv + kvh) * A.max_groups * MAX_QV + qv) * PART_FLOATS;
  const size_t stride = (size_t)MAX_QV * PART_FLOATS;
  float mx = -INFINITY;
  for (int s = tid; s < ng; s += MERGE_THREADS) mx = fmaxf(mx, src[s * stride]);
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) mx = xor_max(mx, o);
  if ((tid & 63) == 0) red[tid >> 6] = mx;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < MERGE_THREADS / 64; ++w) mx = fmaxf(mx, red[w]);
  float L = 0.f, o = 0.f;
  for (int s0 = 0; s0 < ng; s0 += MERGE_CHUNK) {
    __syncthreads();  // red and the previous chunk's weights are consumed
    if (s0 + tid < ng) {
      const float* ps = src + (s0 + tid) * stride;
      const float f = mx == -INFINITY ? 0.f : exp2f(ps[0] - mx);
      fw[tid] = f;
      L = __builtin_fmaf(ps[1], f, L);
    }
    __syncthreads();
    const int n = min(MERGE_CHUNK, ng - s0);
    const float* po = src + s0 * stride + 4 + d;
#pragma unroll 4
    for (int i = part; i < n; i += MERGE_PARTS) o = __builtin_fmaf(fw[i], po[i * stride], o);
  }
#pragma unroll
  for (int s = 1; s < 64; s <<= 1) L = xor_sum(L, s);
  __syncthreads();
  if ((tid & 63) == 0) red[tid >> 6] = L;
  osum[part][d] = o;
  __syncthreads();
  if (part == 0) {
    L = 0.f;
#pragma unroll
    for (int w = 0; w < MERGE_THREADS / 64; ++w) L += red[w];
    o = ((osum[0][d] + osum[1][d]) + osum[2][d]) + osum[3][d];
    A.out[((size_t)r * A.n_heads + h) * HEAD_DIM + d] = L > 0.f ? o / (L * P_SCALE) : 0.f;
  }
}

bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

}  // namespace mk

extern "C" {

size_t mk_q8_attn_workspace_bytes(int n_agents, int max_pages, int n_kv) {
  if (n_agents < 1 || max_pages < 1 || n_kv < 1) return 0;
  const int gpages = mk::ATT_WAVES * mk::pages_per_wave(max_pages);
  const size_t groups = (size_t)(max_pages + gpages - 1) / gpages;
  return (size_t)n_agents * n_kv * groups * mk::MAX_QV * mk::PART_FLOATS * sizeof(float);
}

int mk_q8_attn_decode(const uint16_t* Q, const void* pool, int n_pages,
                      const int32_t* block_table, const int32_t* row_len, int n_agents,
                      int rows_per_agent, int max_pages, int n_heads, int n_kv, float* O,
                      void* workspace, size_t ws_bytes, void* stream) {
  using namespace mk;
  if (!Q || !pool || !block_table || !row_len || !O || !workspace) return MK_EINVAL;
  if (n_pages < 1 || n_agents < 1 || rows_per_agent < 1 || max_pages < 1 || n_kv < 1 ||
      n_heads < n_kv ||
      n_heads % n_kv)
    return MK_EINVAL;
  const int group = n_heads / n_kv;
  if (rows_per_agent * group > MAX_QV) return MK_EINVAL;
  if (!al16(Q) || !al16(pool) || !al16(O) || !al16(workspace)) return MK_EALIGN;
  if (ws_bytes < mk_q8_attn_workspace_bytes(n_agents, max_pages, n_kv)) return MK_EWORKSPACE;
  AttnArgs A;
  A.q = Q;
  A.pool = static_cast<const uint8_t*>(pool);
  A.table = block_table;
  A.row_len = row_len;
  A.part = static_cast<float*>(workspace);
  A.out = O;
  A.n_agents = n_agents;
  A.rows = rows_per_agent;
  A.max_pages = max_pages;
  A.n_heads = n_heads;
  A.n_kv = n_kv;
  A.group = group;
  A.nqv = rows_per_agent * group;
  A.ppw = pages_per_wave(max_pages);
  A.max_groups = (max_pages + ATT_WAVES * A.ppw - 1) / (ATT_WAVES * A.ppw);
  A.n_pages = n_pages;
  A.qk_scale = (float)(1.4426950408889634 / sqrt((double)HEAD_DIM));
  hipStream_t st = static_cast<hipStream_t>(stream);
  const long long blocks = (long long)n_agents * n_kv * A.max_groups;
  if (blocks > 0x7FFFFFFF) return MK_EINVAL;
  if (A.nqv <= 16)
    hipLaunchKernelGGL(q8_attn_kernel<1>, dim3((unsigned)blocks), dim3(ATT_THREADS), 0, st, A);
  else
    hipLaunchKernelGGL(q8_attn_kernel<2>, dim3((unsigned)blocks), dim3(ATT_THREADS), 0, st, A);
  if (hipGetLastError() != hipSuccess) return MK_EHIP;
  hipLaunchKernelGGL(q8_attn_merge, dim3((unsigned)(n_agents * rows_per_agent * n_heads)),
                     dim3(MERGE_THREADS), 0, st, A);
  return hipGetLastError() == hipSuccess ? MK_OK : MK_EHIP;
}

}  // extern "C"
