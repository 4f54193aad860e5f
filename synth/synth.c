/*
 * synth.c - seeded, seekable generator of synthetic Q4_K weight blocks and
 * fp16 activation rows.
 *
 * This module produces INPUTS only. It holds none of the arithmetic of the
 * method under test: it never decodes a block, never dequantizes and never
 * multiplies. Both the GPU path's tests/bench and the CPU oracle consume the
 * bytes it writes; neither imports the other.
 *
 * Distributions (the workload definition of the single-matrix decode GEMM):
 *   d, dmin : binary16 of |z| * 1e-3, z ~ N(0,1), round-to-nearest-even
 *   the 12 scale/min bytes and the 128 nibble bytes : independent uniform
 *             bytes. Every 6-bit scale, 6-bit min and 4-bit quant field of the
 *             Q4_K block is a disjoint set of bits of those bytes, so uniform
 *             bytes give each field the uniform distribution over its range
 *             (0..63 for scales/mins, 0..15 for quants), independently.
 *   activations : binary16 of z, z ~ N(0,1), round-to-nearest-even.
 *
 * Centred blocks (synth_q4k_blocks_centered, for the residual layer walk,
 * whose norms do not remove a common offset): the same draws, then every
 * sub-block gets scale sc = 1 + (2 bits of the original scale bytes) in
 * 1..4 and min m = 15 * sc, and dmin = binary16(|z| * 0.5e-3) from the same
 * normal z as d, so that a weight d*sc*q - dmin*m = d*sc*(q - 7.5) (up to
 * the roundings of d and dmin) has mean about zero over the uniform quants. The 12 scale bytes are packed in the
 * Q4_K layout: bytes 0-3 hold the 6-bit scales of sub-blocks 0-3 and, in
 * bits 6-7, the top bits of the scales of 4-7; bytes 4-7 the same for the
 * mins; bytes 8-11 the low 4 bits of the scale (low nibble) and min (high
 * nibble) of sub-blocks 4-7.
 *
 * Paged q8_0 KV pool (decode attention): page p, KV head h occupies 4352
 * bytes at (p * n_kv + h) * 4352, one int8 quant per value and one binary16
 * scale per token and 32-dim block (as in q8_0), placed as follows (token t,
 * dim d, block b = d / 32; g = t / 4 or (d % 32) / 8 as stated):
 *   K quant (t, d): 1024 * (b / 2) + 16 * (16 * ((d % 32) / 8) + t)
 *                   + 8 * (b % 2) + d % 8
 *   V quant (t, d): 1024 * (2 + d / 64) + 16 * (16 * (t / 4) + d % 16)
 *                   + 4 * ((d / 16) % 4) + t % 4
 *   K scale (t, b): 4096 + 64 * (t / 4) + 2 * (4 * (t % 4) + b)
 *   V scale (t, b): 4096 + 64 * (t / 4) + 32 + 2 * (4 * (t % 4) + b)
 * Quants are uniform bytes; scales are binary16 of |z| * 0.03, z ~ N(0,1).
 * Page-head j (= page * n_kv + head) takes its quant bytes from draws
 * j*512 .. j*512+511 of the stream keyed k ^ A5..A5 (8 bytes each, little
 * end first): byte t*128 + d is K quant (t, d), byte 2048 + d*16 + t is V
 * quant (t, d). Its scales come from the Box-Muller pairs of draws
 * j*64 .. j*64+63 of the stream keyed k ^ 5A..5A: number 4t + b is K scale
 * (t, b), number 64 + 4t + b is V scale (t, b).
 *
 * Random source: SplitMix64 (Steele, Lea & Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014). Output i of the stream with
 * key k is mix(k + (i+1)*0x9E3779B97F4A7C15), where mix is the published
 * 64-bit finalizer. The stream is therefore counter-based: any block or
 * element can be regenerated alone from (key, index).
 *
 * Normals: Box-Muller on one 64-bit draw: u1 = (hi32 + 1) / 2^32 in (0,1],
 * u2 = lo32 / 2^32 in [0,1); r = sqrt(-2 ln u1); z0 = r cos(2 pi u2),
 * z1 = r sin(2 pi u2), all in double precision.
 *
 * Block b of a weight stream uses draws 19b .. 19b+18: draw 0 gives (d, dmin)
 * through Box-Muller, draws 1..18 give the 144 block bytes little-endian,
 * whose first four bytes are then replaced by d and dmin (little-endian
 * binary16). Activation element i uses the Box-Muller pair of draw i/2
 * (z0 for even i, z1 for odd i).
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#define SYNTH_GAMMA 0x9E3779B97F4A7C15ULL
#define SYNTH_BLOCK_BYTES 144
#define SYNTH_DRAWS_PER_BLOCK 19

static uint64_t synth_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

/* Output number i (0-based) of the SplitMix64 stream seeded with key. */
uint64_t synth_draw(uint64_t key, uint64_t i) {
  return synth_mix(key + (i + 1) * SYNTH_GAMMA);
}

/* Key of a sub-stream: three nested draws so distinct (seed, a, b, c) give
 * unrelated streams. */
uint64_t synth_key(uint64_t seed, uint64_t a, uint64_t b, uint64_t c) {
  uint64_t k = synth_draw(seed, a);
  k = synth_draw(k, b);
  return synth_draw(k, c);
}

/* binary16 encoding of a double, round to nearest, ties to even; overflow
 * gives infinity. Used only to encode generated values. */
static uint16_t synth_f64_to_f16(double v) {
  uint16_t sign = 0;
  if (signbit(v)) { sign = 0x8000; v = -v; }
  if (isnan(v)) return (uint16_t)(sign | 0x7E00);
  if (v >= 65520.0) return (uint16_t)(sign | 0x7C00); /* rounds to inf */
  if (v < 0x1p-14) {
    /* subnormal range: value = n * 2^-24, n in 0..1024 (1024 = smallest normal) */
    double n = v * 0x1p24;
    double fl = floor(n);
    double frac = n - fl;
    uint32_t r = (uint32_t)fl;
    if (frac > 0.5 || (frac == 0.5 && (r & 1))) r++;
    return (uint16_t)(sign | r); /* r == 1024 encodes 2^-14 exactly */
  }
  int e;
  double m = frexp(v, &e);            /* v = m * 2^e, m in [0.5,1) */
  double n = ldexp(m, 11);            /* 11 significant bits: n in [1024,2048) */
  double fl = floor(n);
  double frac = n - fl;
  uint32_t r = (uint32_t)fl;
  if (frac > 0.5 || (frac == 0.5 && (r & 1))) r++;
  int exp16 = e - 1 + 15;             /* v in [2^(e-1), 2^e) */
  if (r == 2048) { r = 1024; exp16++; }
  if (exp16 >= 31) return (uint16_t)(sign | 0x7C00);
  return (uint16_t)(sign | ((uint32_t)exp16 << 10) | (r - 1024));
}

static void synth_normal_pair(uint64_t w, double* z0, double* z1) {
  double u1 = ((double)(w >> 32) + 1.0) * 0x1p-32;
  double u2 = (double)(w & 0xFFFFFFFFULL) * 0x1p-32;
  double r = sqrt(-2.0 * log(u1));
  double a = 6.283185307179586476925286766559 * u2;
  *z0 = r * cos(a);
  *z1 = r * sin(a);
}

/* Write blocks [b0, b0+nb) of the weight stream `key` to out (nb*144 bytes). */
void synth_q4k_blocks(uint64_t key, uint64_t b0, uint64_t nb, uint8_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < (int64_t)nb; ++i) {
    uint64_t b = b0 + (uint64_t)i;
    uint8_t* blk = out + (size_t)i * SYNTH_BLOCK_BYTES;
    uint64_t base = b * SYNTH_DRAWS_PER_BLOCK;
    for (int t = 0; t < 18; ++t) {
      uint64_t w = synth_draw(key, base + 1 + (uint64_t)t);
      for (int j = 0; j < 8; ++j) blk[8 * t + j] = (uint8_t)(w >> (8 * j));
    }
    double z0, z1;
    synth_normal_pair(synth_draw(key, base), &z0, &z1);
    uint16_t d = synth_f64_to_f16(fabs(z0) * 1e-3);
    uint16_t dmin = synth_f64_to_f16(fabs(z1) * 1e-3);
    blk[0] = (uint8_t)d; blk[1] = (uint8_t)(d >> 8);
    blk[2] = (uint8_t)dmin; blk[3] = (uint8_t)(dmin >> 8);
  }
}

/* As synth_q4k_blocks, with centred scales and mins (see the header). */
void synth_q4k_blocks_centered(uint64_t key, uint64_t b0, uint64_t nb, uint8_t* out) {
  synth_q4k_blocks(key, b0, nb, out);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < (int64_t)nb; ++i) {
    uint8_t* blk = out + (size_t)i * SYNTH_BLOCK_BYTES;
    /* dmin from the same normal as d, halved before the rounding */
    double z0, z1;
    synth_normal_pair(synth_draw(key, (b0 + (uint64_t)i) * SYNTH_DRAWS_PER_BLOCK), &z0, &z1);
    const uint16_t dmin = synth_f64_to_f16(fabs(z0) * 0.5e-3);
    blk[2] = (uint8_t)dmin;
    blk[3] = (uint8_t)(dmin >> 8);
    /* two random bits per sub-block from the (uniform) original scale bytes */
    uint8_t* s12 = blk + 4;
    const unsigned r = (unsigned)s12[0] | ((unsigned)s12[1] << 8);
    int sc[8], mn[8];
    for (int j = 0; j < 8; ++j) {
      sc[j] = 1 + (int)((r >> (2 * j)) & 3u);
      mn[j] = 15 * sc[j];
    }
    for (int j = 0; j < 4; ++j) {
      s12[j] = (uint8_t)((sc[j] & 63) | ((sc[j + 4] >> 4) << 6));
      s12[j + 4] = (uint8_t)((mn[j] & 63) | ((mn[j + 4] >> 4) << 6));
      s12[j + 8] = (uint8_t)((sc[j + 4] & 15) | ((mn[j + 4] & 15) << 4));
    }
  }
}

/* Rows [n0, n0+nrows) of a centred (N, K) matrix. */
void synth_q4k_rows_centered(uint64_t key, int64_t K, int64_t n0, int64_t nrows, uint8_t* out) {
  uint64_t kb = (uint64_t)(K / 256);
  synth_q4k_blocks_centered(key, (uint64_t)n0 * kb, (uint64_t)nrows * kb, out);
}

/* Write the blocks of whole weight rows [n0, n0+nrows) of an (N, K) matrix
 * whose row n holds K/256 consecutive blocks. */
void synth_q4k_rows(uint64_t key, int64_t K, int64_t n0, int64_t nrows, uint8_t* out) {
  uint64_t kb = (uint64_t)(K / 256);
  synth_q4k_blocks(key, (uint64_t)n0 * kb, (uint64_t)nrows * kb, out);
}

/* Write activation elements [i0, i0+n) of stream `key` as binary16 bits. */
void synth_f16_normal(uint64_t key, uint64_t i0, uint64_t n, uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < (int64_t)n; ++j) {
    uint64_t i = i0 + (uint64_t)j;
    double z0, z1;
    synth_normal_pair(synth_draw(key, i >> 1), &z0, &z1);
    out[j] = synth_f64_to_f16((i & 1) ? z1 : z0);
  }
}

/* The Box-Muller normals behind activation elements [i0, i0+n) of stream
 * `key`, before the binary16 rounding (for testing the encoding). */
void synth_normals(uint64_t key, uint64_t i0, uint64_t n, double* out) {
  for (uint64_t j = 0; j < n; ++j) {
    uint64_t i = i0 + j;
    double z0, z1;
    synth_normal_pair(synth_draw(key, i >> 1), &z0, &z1);
    out[j] = (i & 1) ? z1 : z0;
  }
}

/* Q6_K rows [n0, n0+nrows) of an N x K matrix (GGUF Q6_K blocks of 210
 * bytes: ql[128], qh[64], int8 scales[16], binary16 d). Block b (= row * K/256
 * + block in row) takes bytes 0..207 (quants and scales, uniform) from draws
 * 27b .. 27b+25 of the stream keyed k ^ 6666..66 (8 bytes each, little end
 * first), and d = binary16 of |z| * 2^-14 with z the first normal of the
 * Box-Muller pair of draw 27b + 26. */
void synth_q6k_rows(uint64_t key, int64_t K, int64_t n0, int64_t nrows, uint8_t* out) {
  const uint64_t k6 = key ^ 0x6666666666666666ULL;
  const int64_t nb = K / 256;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < nrows * nb; ++i) {
    const uint64_t b = (uint64_t)((n0 + i / nb) * nb + i % nb);
    uint8_t* blk = out + (size_t)i * 210;
    for (int t = 0; t < 208; ++t) blk[t] = (uint8_t)(synth_draw(k6, 27 * b + (uint64_t)(t >> 3)) >> (8 * (t & 7)));
    double z0, z1;
    synth_normal_pair(synth_draw(k6, 27 * b + 26), &z0, &z1);
    const uint16_t d = synth_f64_to_f16(fabs(z0) * 0x1p-14);
    blk[208] = (uint8_t)d;
    blk[209] = (uint8_t)(d >> 8);
  }
}

/* Fill n_pages pages of a paged q8_0 KV pool with n_kv heads (layout above). */
void synth_q8_pool(uint64_t key, int64_t n_pages, int64_t n_kv, uint8_t* out) {
  const uint64_t kq = key ^ 0xA5A5A5A5A5A5A5A5ULL, ks = key ^ 0x5A5A5A5A5A5A5A5AULL;
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < n_pages * n_kv; ++j) {
    uint8_t* ph = out + (size_t)j * 4352;
    for (int i = 0; i < 4096; ++i) {  /* 2048 K quant bytes, then 2048 V quant bytes */
      const uint8_t q = (uint8_t)(synth_draw(kq, (uint64_t)j * 512 + (uint64_t)(i >> 3)) >> (8 * (i & 7)));
      int off;
      if (i < 2048) {
        const int t = i / 128, d = i % 128, b = d / 32;
        off = 1024 * (b / 2) + 16 * (16 * ((d % 32) / 8) + t) + 8 * (b % 2) + d % 8;
      } else {
        const int d = (i - 2048) / 16, t = (i - 2048) % 16;
        off = 1024 * (2 + d / 64) + 16 * (16 * (t / 4) + d % 16) + 4 * ((d / 16) % 4) + t % 4;
      }
      ph[off] = q;
    }
    for (int i = 0; i < 128; ++i) {  /* 64 K scales, then 64 V scales */
      double z0, z1;
      synth_normal_pair(synth_draw(ks, (uint64_t)j * 64 + (uint64_t)(i >> 1)), &z0, &z1);
      const uint16_t sc = synth_f64_to_f16(fabs((i & 1) ? z1 : z0) * 0.03);
      const int n = i % 64, t = n / 4, b = n % 4;
      uint8_t* dst = ph + 4096 + 64 * (t / 4) + (i < 64 ? 0 : 32) + 2 * (4 * (t % 4) + b);
      dst[0] = (uint8_t)sc;
      dst[1] = (uint8_t)(sc >> 8);
    }
  }
}
