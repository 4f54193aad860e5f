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
// Work split: one workgroup of 4 waves per (agent, KV head, group of 64
// pages); wave w takes 16 consecutive pages of the group. All R x group
// query vectors of the (agent, KV head) ride in one wave (up to 32: two
// 16-column MFMA tiles), so every K and V byte is read once per step.
//
// Per page (16 tokens), with MFMA (f16 in, fp32 accumulate):
//   scores  S^T[t][q] = sum_u ks[t][u] * (Kq_u . Q_u)  - four 16x16x32 MFMAs
//           per query tile, one per 32-dim q8_0 block u, the int8 quants
//           entering exactly and each block's scale applied to its product;
//   softmax online over the pages, in the log2 domain, per query column;
//   values  O^T[d][q] += sigma * (Vq^T . B), B[t][q] = p[t][q] * vs[t][b] /
//           sigma * 2^12 split into binary16 hi + lo (two 16x16x16 MFMAs per
//           16-dim tile), sigma a power of two at least the page's largest V
//           scale, so B stays in binary16's normal range; the 2^12 is taken
//           out at the end.
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
constexpr int PAGES_PER_WAVE = 16;
constexpr int PAGES_PER_GROUP = PAGES_PER_WAVE * ATT_WAVES;
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
  float qk_scale;           // log2(e) / sqrt(128)
};

__device__ __forceinline__ float xor_max(float v, int m) {
  return fmaxf(v, __shfl_xor(v, m, 64));
}
__device__ __forceinline__ float xor_sum(float v, int m) { return v + __shfl_xor(v, m, 64); }

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

__global__ void __launch_bounds__(ATT_THREADS) q8_attn_kernel(AttnArgs A) {
  __shared__ float st_s[ATT_WAVES][2][64][2];             // per wave: (max, sum) per lane
  __shared__ floatx4 acc_s[ATT_WAVES][2][8][64];          // per wave: the 16 output tiles
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int c = lane & 15, g = lane >> 4;
  const int grp = blockIdx.x % A.max_groups;
  const int kvh = (blockIdx.x / A.max_groups) % A.n_kv;
  const int a = blockIdx.x / (A.max_groups * A.n_kv);
  const int len_a = agent_len(A, a);
  const int npages = (len_a + PAGE_TOKENS - 1) / PAGE_TOKENS;
  if (grp * PAGES_PER_GROUP >= npages) return;  // nothing here (uniform per workgroup)
  const int p0 = grp * PAGES_PER_GROUP + wave * PAGES_PER_WAVE;
  const int p1 = min(p0 + PAGES_PER_WAVE, npages);

  // query operands (B of the score MFMA): query vector 16 qt + c, dims
  // 32 u + 8 g .. +7; past the agent's query vectors: zeros, length 0
  half8v qop[2][4];
  int qlen[2];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const int qv = 16 * qt + c;
    const bool live = qv < A.nqv;
    const int j = live ? qv / A.group : 0, hh = live ? qv % A.group : 0;
    const int row = a * A.rows + j, head = kvh * A.group + hh;
    qlen[qt] = live ? row_tokens(A, row) : 0;
    const uint16_t* qp = A.q + ((size_t)row * A.n_heads + head) * HEAD_DIM;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      u32x4 v = live ? *reinterpret_cast<const u32x4*>(qp + 32 * u + 8 * g) : u32x4{0u, 0u, 0u, 0u};
      qop[qt][u] = __builtin_bit_cast(half8v, v);
    }
  }

  float m[2] = {-INFINITY, -INFINITY}, lsum[2] = {0.f, 0.f};
  floatx4 acc[2][8];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt)
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) acc[qt][dt] = floatx4{0.f, 0.f, 0.f, 0.f};

  const int32_t* tab = A.table + (size_t)a * A.max_pages;
  for (int p = p0; p < p1; ++p) {
    const int page = min(max(tab[p], 0), A.n_pages - 1);  // in range whatever the table holds
    const uint8_t* ph = A.pool + ((size_t)page * A.n_kv + kvh) * PAGE_HEAD_BYTES;
    // K quants of token c, dims 32u + 8g .. +7; scales of tokens 4g..4g+3
    // (all four blocks); V quants of dims 16 dt + c, tokens 4g .. 4g+3; V
    // scales of tokens 4g .. 4g+3
    u32x2 kq[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      kq[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(ph + c * 128 + 32 * u + 8 * g));
    const u32x4 ks0 = *reinterpret_cast<const u32x4*>(ph + 2048 + 32 * g);
    const u32x4 ks1 = *reinterpret_cast<const u32x4*>(ph + 2048 + 32 * g + 16);
    uint32_t vq[8];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
      vq[dt] = __builtin_nontemporal_load(
          reinterpret_cast<const uint32_t*>(ph + 2176 + (16 * dt + c) * 16 + 4 * g));
    const u32x4 vs0 = *reinterpret_cast<const u32x4*>(ph + 4224 + 32 * g);
    const u32x4 vs1 = *reinterpret_cast<const u32x4*>(ph + 4224 + 32 * g + 16);
    // ks[r][u]: token 4g + r, block u
    float ks[4][4], vs[4][4];
    {
      const uint32_t kw[8] = {ks0.x, ks0.y, ks0.z, ks0.w, ks1.x, ks1.y, ks1.z, ks1.w};
      const uint32_t vw[8] = {vs0.x, vs0.y, vs0.z, vs0.w, vs1.x, vs1.y, vs1.z, vs1.w};
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int i = 4 * r + u;
          ks[r][u] = (float)bit_cast_<_Float16>((uint16_t)(kw[i >> 1] >> (16 * (i & 1))));
          vs[r][u] = (float)bit_cast_<_Float16>((uint16_t)(vw[i >> 1] >> (16 * (i & 1))));
        }
    }
    // K quants as exact binary16 (A operand of the score MFMA)
    half8v ka[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t w[2] = {kq[u].x, kq[u].y};
#pragma unroll
      for (int e = 0; e < 8; ++e)
        ka[u][e] = (_Float16)(float)(int8_t)(w[e >> 2] >> (8 * (e & 3)));
    }
    // the page's V scale bound: a power of two >= every scale of the page
    float vmax = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int u = 0; u < 4; ++u) vmax = fmaxf(vmax, vs[r][u]);
    vmax = xor_max(xor_max(vmax, 16), 32);  // the page's 16 tokens: lane groups g = 0..3
    const uint32_t vb = __builtin_bit_cast(uint32_t, vmax);
    const float sigma = vmax > 0.f ? __builtin_bit_cast(float, (vb + 0x007FFFFFu) & 0xFF800000u) : 1.f;
    const float bscale = P_SCALE / sigma;

    const int tok0 = p * PAGE_TOKENS + 4 * g;  // this lane's first token
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      floatx4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const floatx4 su =
            __builtin_amdgcn_mfma_f32_16x16x32_f16(ka[u], qop[qt][u], floatx4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) s[r] = __builtin_fmaf(ks[r][u], su[r], s[r]);
      }
      float pv[4];
      float mp = -INFINITY;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        pv[r] = tok0 + r < qlen[qt] ? s[r] * A.qk_scale : -INFINITY;
        mp = fmaxf(mp, pv[r]);
      }
      mp = xor_max(xor_max(mp, 16), 32);
      const float mn = fmaxf(m[qt], mp);
      float alpha = 1.f, ps = 0.f;
      if (mn != -INFINITY) {
        alpha = exp2f(m[qt] - mn);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          pv[r] = exp2f(pv[r] - mn);
          ps += pv[r];
        }
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) pv[r] = 0.f;
      }
      ps = xor_sum(xor_sum(ps, 16), 32);
      lsum[qt] = __builtin_fmaf(lsum[qt], alpha, ps);
      m[qt] = mn;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const int b = dt >> 1;
        half4v bh, bl;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float v = pv[r] * vs[r][b] * bscale;
          const _Float16 h = (_Float16)v;
          bh[r] = h;
          bl[r] = (_Float16)(v - (float)h);
        }
        half4v av;
#pragma unroll
        for (int r = 0; r < 4; ++r) av[r] = (_Float16)(float)(int8_t)(vq[dt] >> (8 * r));
        floatx4 t = __builtin_amdgcn_mfma_f32_16x16x16f16(av, bh, floatx4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
        t = __builtin_amdgcn_mfma_f32_16x16x16f16(av, bl, t, 0, 0, 0);
        const floatx4 al = {alpha, alpha, alpha, alpha};
        const floatx4 sg = {sigma, sigma, sigma, sigma};
        acc[qt][dt] = __builtin_elementwise_fma(sg, t, acc[qt][dt] * al);
      }
    }
  }

  // merge the four waves in LDS (fixed order), then one partial per workgroup
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    st_s[wave][qt][lane][0] = m[qt];
    st_s[wave][qt][lane][1] = lsum[qt];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) acc_s[wave][qt][dt][lane] = acc[qt][dt];
  }
  __syncthreads();
  // thread: (query tile qt = wave >> 1, half of the d tiles = wave & 1), lane
  const int qt = wave >> 1, dh = wave & 1;
  float mx = -INFINITY;
#pragma unroll
  for (int w = 0; w < ATT_WAVES; ++w) mx = fmaxf(mx, st_s[w][qt][lane][0]);
  float L = 0.f;
  floatx4 o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int w = 0; w < ATT_WAVES; ++w) {
    const float mw = st_s[w][qt][lane][0];
    const float f = mx == -INFINITY ? 0.f : exp2f(mw - mx);
    L = __builtin_fmaf(st_s[w][qt][lane][1], f, L);
    const floatx4 ff = {f, f, f, f};
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = __builtin_elementwise_fma(ff, acc_s[w][qt][4 * dh + i][lane], o[i]);
  }
  const int qv = 16 * qt + c;
  if (qv < A.nqv) {
    float* dst = A.part + ((((size_t)a * A.n_kv + kvh) * A.max_groups + grp) * MAX_QV + qv) * PART_FLOATS;
    if (dh == 0 && g == 0) {
      dst[0] = mx;
      dst[1] = L;
    }
    // tile dt holds dims 16 dt + 4 g .. +3 of query qv (scaled by 2^12)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<floatx4*>(dst + 4 + 16 * (4 * dh + i) + 4 * g) = o[i];
  }
}

// One block per (row, head), one thread per output dim: add the partials of
// the row's agent and KV head in group order.
__global__ void __launch_bounds__(HEAD_DIM) q8_attn_merge(AttnArgs A) {
  const int r = blockIdx.x / A.n_heads, h = blockIdx.x % A.n_heads, d = threadIdx.x;
  const int a = r / A.rows, j = r % A.rows;
  const int kvh = h / A.group, qv = j * A.group + h % A.group;
  const int npages = (agent_len(A, a) + PAGE_TOKENS - 1) / PAGE_TOKENS;
  const int ng = (npages + PAGES_PER_GROUP - 1) / PAGES_PER_GROUP;
  const float* src = A.part + (((size_t)a * A.n_kv + kvh) * A.max_groups * MAX_QV + qv) * PART_FLOATS;
  const size_t stride = (size_t)MAX_QV * PART_FLOATS;
  float mx = -INFINITY;
  for (int s = 0; s < ng; ++s) mx = fmaxf(mx, src[s * stride]);
  float L = 0.f, o = 0.f;
  for (int s = 0; s < ng; ++s) {
    const float* ps = src + s * stride;
    const float f = mx == -INFINITY ? 0.f : exp2f(ps[0] - mx);
    L = __builtin_fmaf(ps[1], f, L);
    o = __builtin_fmaf(ps[4 + d], f, o);
  }
  A.out[((size_t)r * A.n_heads + h) * HEAD_DIM + d] = L > 0.f ? o / (L * P_SCALE) : 0.f;
}

bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

}  // namespace mk

extern "C" {

size_t mk_q8_attn_workspace_bytes(int n_agents, int max_pages, int n_kv) {
  if (n_agents < 1 || max_pages < 1 || n_kv < 1) return 0;
  const size_t groups = (size_t)(max_pages + mk::PAGES_PER_GROUP - 1) / mk::PAGES_PER_GROUP;
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
  A.max_groups = (max_pages + PAGES_PER_GROUP - 1) / PAGES_PER_GROUP;
  A.n_pages = n_pages;
  A.qk_scale = (float)(1.4426950408889634 / sqrt((double)HEAD_DIM));
  hipStream_t st = static_cast<hipStream_t>(stream);
  const long long blocks = (long long)n_agents * n_kv * A.max_groups;
  if (blocks > 0x7FFFFFFF) return MK_EINVAL;
  hipLaunchKernelGGL(q8_attn_kernel, dim3((unsigned)blocks), dim3(ATT_THREADS), 0, st, A);
  if (hipGetLastError() != hipSuccess) return MK_EHIP;
  hipLaunchKernelGGL(q8_attn_merge, dim3((unsigned)(n_agents * rows_per_agent * n_heads)),
                     dim3(HEAD_DIM), 0, st, A);
  return hipGetLastError() == hipSuccess ? MK_OK : MK_EHIP;
}

}  // extern "C"
