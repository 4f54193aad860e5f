/*
 * q4k_oracle.c - plain, slow fp64 CPU reference of the Q4_K weight-streaming
 * decode GEMM. TEST INFRASTRUCTURE ONLY: only the test suite, the smoke check
 * and the CPU-baseline leg of the benchmark may load it. The product path
 * never calls it and shares no code with it.
 *
 * What it computes (the multi-agent decode step of the OpenJet post, "RTX 3090
 * one card, four coding agents", paragraph on how parallel decoding works:
 * every agent's rows are stacked into one batch and each weight, read once,
 * multiplies all of them):
 *
 *   y[m][n] = sum_k x[m][k] * w[n][k]          (Y = X * W^T)
 *   S[m][n] = sum_k |x[m][k] * w[n][k]|        (the per-element error scale)
 *
 * with w the exact dequantized Q4_K weight. Every step is done in double
 * precision with k in increasing order; no blocking, no reordering.
 *
 * Q4_K block (144 bytes per 256 weights, the public GGUF k-quant layout; the
 * pages name the format only as "Q4_K_M"):
 *   bytes 0-1   d      (binary16, little-endian)
 *   bytes 2-3   dmin   (binary16, little-endian)
 *   bytes 4-15  twelve bytes of packed 6-bit scales sc[0..7] and mins m[0..7]
 *   bytes 16-143 128 bytes of 4-bit quants
 *   weight t (0..255) of the block, in sub-block j = t/32:
 *     w = d * sc[j] * q[t] - dmin * m[j]
 *
 * Every dequantized weight is exact in double: d has an 11-bit significand,
 * sc[j]*q[t] <= 945 has 10 bits, dmin*m[j] has 17 bits, so both products and
 * their difference fit in 53 bits.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>

#define ORACLE_BLOCK_BYTES 144
#define ORACLE_QK 256

/* binary16 -> double, decoded bit by bit:
 *   exponent field 0   : subnormal, value = mantissa * 2^-24
 *   exponent field 31  : infinity (mantissa 0) or NaN
 *   otherwise          : (1024 + mantissa) * 2^(exponent - 25)           */
double oracle_f16_to_f64(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 31;
  int mant = h & 1023;
  double v;
  if (e == 0) {
    v = ldexp((double)mant, -24);
  } else if (e == 31) {
    v = mant ? NAN : INFINITY;
  } else {
    v = ldexp((double)(1024 + mant), e - 25);
  }
  return sign ? -v : v;
}

/* double -> binary16 bits, round to nearest with ties to even; magnitudes
 * that round beyond 65504 give infinity. The spacing of binary16 values at
 * |v| is 2^-24 below 2^-14 and 2^(e-11) for |v| in [2^(e-1), 2^e) above it;
 * the neighbour is picked from the exact remainder. */
uint16_t oracle_f64_to_f16(double v) {
  if (isnan(v)) return 0x7E00;
  uint16_t sign = signbit(v) ? 0x8000 : 0;
  double a = fabs(v);
  /* 65504 is the largest finite value; 65520, the midpoint to 65536, ties to
   * the even side, which is the overflow. */
  if (a >= 65520.0) return sign | 0x7C00;
  double ulp;
  if (a < 0x1p-14) {
    ulp = 0x1p-24;
  } else {
    int e;
    frexp(a, &e);
    ulp = ldexp(1.0, e - 11);
  }
  double n = floor(a / ulp);   /* exact: division by a power of two */
  double rem = a - n * ulp;    /* exact */
  if (rem > 0.5 * ulp || (rem == 0.5 * ulp && fmod(n, 2.0) != 0.0)) n += 1.0;
  double pick = n * ulp;
  if (pick < 0x1p-14) return sign | (uint16_t)(pick * 0x1p24);
  int e;
  double m = frexp(pick, &e); /* pick = m * 2^e, m in [0.5, 1) */
  int ef = e - 1 + 15;
  int mant = (int)(ldexp(m, 11) - 1024.0);
  return sign | (uint16_t)(ef << 10) | (uint16_t)mant;
}

/* Split the 12 packed bytes into the eight 6-bit scales and eight 6-bit mins.
 * Sub-blocks 0..3 keep their scale in the low 6 bits of bytes 0..3 and their
 * min in the low 6 bits of bytes 4..7. Sub-blocks 4..7 keep the low 4 bits of
 * scale and min in the low and high nibble of bytes 8..11, and the top 2 bits
 * in the top 2 bits of bytes 0..3 (scale) and 4..7 (min). */
void oracle_unpack_scales(const uint8_t* s12, int sc[8], int mn[8]) {
  for (int j = 0; j < 4; ++j) {
    sc[j] = s12[j] & 63;
    mn[j] = s12[j + 4] & 63;
  }
  for (int j = 4; j < 8; ++j) {
    int low4_sc = s12[j + 4] & 15;
    int low4_m = s12[j + 4] >> 4;
    int top2_sc = s12[j - 4] >> 6;
    int top2_m = s12[j] >> 6;
    sc[j] = low4_sc | (top2_sc << 4);
    mn[j] = low4_m | (top2_m << 4);
  }
}

/* Quants: byte i (0..31) of 32-byte chunk c (0..3) holds weight 64c+i in its
 * low nibble (sub-block 2c) and weight 64c+32+i in its high nibble
 * (sub-block 2c+1). */
void oracle_unpack_quants(const uint8_t* qs128, int q[256]) {
  for (int c = 0; c < 4; ++c) {
    for (int i = 0; i < 32; ++i) {
      uint8_t b = qs128[32 * c + i];
      q[64 * c + i] = b & 15;
      q[64 * c + 32 + i] = b >> 4;
    }
  }
}

/* Decode one block into its fields. */
void oracle_decode_block(const uint8_t* blk, double* d, double* dmin, int sc[8], int mn[8],
                         int q[256]) {
  uint16_t hd = (uint16_t)(blk[0] | (blk[1] << 8));
  uint16_t hm = (uint16_t)(blk[2] | (blk[3] << 8));
  *d = oracle_f16_to_f64(hd);
  *dmin = oracle_f16_to_f64(hm);
  oracle_unpack_scales(blk + 4, sc, mn);
  oracle_unpack_quants(blk + 16, q);
}

/* Dequantize one weight row of K values (K/256 consecutive blocks). */
void oracle_dequant_row(const uint8_t* row, int64_t K, double* w) {
  int sc[8], mn[8], q[256];
  double d, dmin;
  for (int64_t kb = 0; kb < K / ORACLE_QK; ++kb) {
    oracle_decode_block(row + kb * ORACLE_BLOCK_BYTES, &d, &dmin, sc, mn, q);
    for (int t = 0; t < ORACLE_QK; ++t) {
      int j = t / 32;
      w[kb * ORACLE_QK + t] = d * (double)sc[j] * (double)q[t] - dmin * (double)mn[j];
    }
  }
}

void oracle_dequant_rows(const uint8_t* W, int64_t nrows, int64_t K, double* w) {
  int64_t row_bytes = K / ORACLE_QK * ORACLE_BLOCK_BYTES;
  for (int64_t n = 0; n < nrows; ++n) oracle_dequant_row(W + n * row_bytes, K, w + n * K);
}

void oracle_standardize(const double* v, int64_t M, int64_t N, double eps, double* t);

/* y = xd * W^T and S = |xd| * |W|^T for double activations xd [M][K]: the
 * product both references below share. Threads split the columns; each
 * column is dequantized once into a private double buffer, then every row m
 * is a plain in-order dot product. */
typedef void (*row_decoder)(const uint8_t* row, int64_t K, double* w);

static int gemm_f64_rows(const uint8_t* W, int64_t row_bytes, row_decoder dequant,
                         const double* xd, int64_t M, int64_t ncols, int64_t K, double* y,
                         double* S) {
  int err = 0;
#pragma omp parallel
  {
    double* w = (double*)malloc(sizeof(double) * (size_t)K);
    if (!w) {
#pragma omp atomic write
      err = -2;
    }
#pragma omp for schedule(dynamic, 4)
    for (int64_t n = 0; n < ncols; ++n) {
      if (!w) continue;
      dequant(W + n * row_bytes, K, w);
      for (int64_t m = 0; m < M; ++m) {
        const double* xm = xd + m * K;
        double acc = 0.0, sabs = 0.0;
        for (int64_t k = 0; k < K; ++k) {
          double p = w[k] * xm[k];
          acc += p;
          sabs += fabs(p);
        }
        y[m * ncols + n] = acc;
        S[m * ncols + n] = sabs;
      }
    }
    free(w);
  }
  return err;
}

static int gemm_f64(const uint8_t* W, const double* xd, int64_t M, int64_t ncols, int64_t K,
                    double* y, double* S) {
  return gemm_f64_rows(W, K / ORACLE_QK * ORACLE_BLOCK_BYTES, oracle_dequant_row, xd, M, ncols,
                       K, y, S);
}

/* Reference GEMM. W holds `ncols` weight rows (the output columns to check),
 * X is fp16 [M][K] row-major (bits), outputs y and S are double [M][ncols]. */
int oracle_gemm(const uint8_t* W, const uint16_t* X, int64_t M, int64_t ncols, int64_t K,
                double* y, double* S) {
  if (K % ORACLE_QK) return -1;
  double* xd = (double*)malloc(sizeof(double) * (size_t)(M * K));
  if (!xd) return -2;
  for (int64_t i = 0; i < M * K; ++i) xd[i] = oracle_f16_to_f64(X[i]);
  int err = gemm_f64(W, xd, M, ncols, K, y, S);
  free(xd);
  return err;
}

/* Reference for one matrix of the layer walk: the product of the row-wise
 * standardized binary16 input with the weights,
 *   y[m][n] = sum_k t[m][k] * w[n][k],   S[m][n] = sum_k |t[m][k] * w[n][k]|,
 *   t[m][k] = (x[m][k] - mean_m) / sqrt(var_m + eps),
 * mean and (population) variance over the K values of row m of x, all in
 * double: the standardization is exact, never rounded to binary16. */
int oracle_gemm_std(const uint8_t* W, const uint16_t* X, int64_t M, int64_t ncols, int64_t K,
                    double eps, double* y, double* S) {
  if (K % ORACLE_QK) return -1;
  double* xd = (double*)malloc(sizeof(double) * (size_t)(M * K));
  double* t = (double*)malloc(sizeof(double) * (size_t)(M * K));
  if (!xd || !t) {
    free(xd);
    free(t);
    return -2;
  }
  for (int64_t i = 0; i < M * K; ++i) xd[i] = oracle_f16_to_f64(X[i]);
  oracle_standardize(xd, M, K, eps, t);
  int err = gemm_f64(W, t, M, ncols, K, y, S);
  free(xd);
  free(t);
  return err;
}

/* Mean and 1 / sqrt(var + eps) of each row of v [M][N], the (population)
 * variance taken about the mean, in double. */
void oracle_row_moments(const double* v, int64_t M, int64_t N, double eps, double* mean_out,
                        double* inv_out) {
  for (int64_t m = 0; m < M; ++m) {
    const double* r = v + m * N;
    double mean = 0.0;
    for (int64_t n = 0; n < N; ++n) mean += r[n];
    mean /= (double)N;
    double var = 0.0;
    for (int64_t n = 0; n < N; ++n) var += (r[n] - mean) * (r[n] - mean);
    var /= (double)N;
    mean_out[m] = mean;
    inv_out[m] = 1.0 / sqrt(var + eps);
  }
}

/* The row-wise standardization every matrix of the layer walk applies to its
 * input:
 *   t[m][n] = (v[m][n] - mean_m) / sqrt(var_m + eps)
 * with mean and (population) variance over the row's N values, in double. */
void oracle_standardize(const double* v, int64_t M, int64_t N, double eps, double* t) {
  for (int64_t m = 0; m < M; ++m) {
    double mean, inv;
    oracle_row_moments(v + m * N, 1, N, eps, &mean, &inv);
    for (int64_t n = 0; n < N; ++n) t[m * N + n] = (v[m * N + n] - mean) * inv;
  }
}

/* The size of the two terms of the factored weight, against which a product
 * that multiplies d * sc[j] * q and dmin * m[j] separately (and subtracts)
 * keeps its error:
 *   F[m][n] = r[m] * ( sum_k (|d sc[j] q[k]| + |dmin m[j]|) * |x[m][k]|
 *                      + |mean[m] * sum_k w[n][k]| )
 * for binary16 X [M][K]; mean and r are per row (mean 0 and r 1 for a plain
 * product, the input's mean and 1 / sqrt(var + eps) for a matrix of the walk,
 * whose products are taken with x and standardized after). F >= sum_k
 * |w x| * r whenever the mean is 0 (|w| <= |d sc q| + |dmin m|), with
 * equality when no weight's two terms have opposite signs. */
int oracle_factored_size(const uint8_t* W, const uint16_t* X, int64_t M, int64_t ncols, int64_t K,
                         const double* mean, const double* r, double* F) {
  if (K % ORACLE_QK) return -1;
  const int64_t row_bytes = K / ORACLE_QK * ORACLE_BLOCK_BYTES;
  int err = 0;
#pragma omp parallel
  {
    double* a = (double*)malloc(sizeof(double) * (size_t)K); /* |d sc q| + |dmin m| */
    double* xa = (double*)malloc(sizeof(double) * (size_t)(M * K));
    if (!a || !xa) {
#pragma omp atomic write
      err = -2;
    } else {
      for (int64_t i = 0; i < M * K; ++i) xa[i] = fabs(oracle_f16_to_f64(X[i]));
    }
#pragma omp for schedule(dynamic, 4)
    for (int64_t n = 0; n < ncols; ++n) {
      if (!a || !xa) continue;
      const uint8_t* row = W + n * row_bytes;
      double wsum = 0.0;
      int sc[8], mn[8], q[256];
      double d, dmin;
      for (int64_t kb = 0; kb < K / ORACLE_QK; ++kb) {
        oracle_decode_block(row + kb * ORACLE_BLOCK_BYTES, &d, &dmin, sc, mn, q);
        for (int t = 0; t < ORACLE_QK; ++t) {
          const int j = t / 32;
          const double main = d * (double)sc[j] * (double)q[t], off = dmin * (double)mn[j];
          a[kb * ORACLE_QK + t] = fabs(main) + fabs(off);
          wsum += main - off;
        }
      }
      for (int64_t m = 0; m < M; ++m) {
        double acc = 0.0;
        for (int64_t k = 0; k < K; ++k) acc += a[k] * xa[m * K + k];
        F[m * ncols + n] = r[m] * (acc + fabs(mean[m] * wsum));
      }
    }
    free(a);
    free(xa);
  }
  return err;
}

/* The residual layer walk: the RMSNorm scale of each row of the fp32
 * residual h [M][N], r[m] = 1 / sqrt(sum_n h[m][n]^2 / N + eps) (the norm's
 * per-column weight is applied before the binary16 cast of the input, the
 * row scale after the product). */
void oracle_rms_inv(const double* h, int64_t M, int64_t N, double eps, double* r) {
  for (int64_t m = 0; m < M; ++m) {
    double ss = 0.0;
    for (int64_t n = 0; n < N; ++n) ss += h[m * N + n] * h[m * N + n];
    r[m] = 1.0 / sqrt(ss / (double)N + eps);
  }
}

/* Reference for a normed matrix of the residual walk: y = r[m] * x * W^T
 * and S = r[m] * |x| * |W|^T, with x the binary16 input [M][K] and r the
 * RMSNorm scale of the residual row (oracle_rms_inv). The product is taken
 * on the row-scaled input, r[m] * x[m][k]. */
int oracle_gemm_rms(const uint8_t* W, const uint16_t* X, int64_t M, int64_t ncols, int64_t K,
                    const double* r, double* y, double* S) {
  if (K % ORACLE_QK) return -1;
  double* xd = (double*)malloc(sizeof(double) * (size_t)(M * K));
  if (!xd) return -2;
  for (int64_t m = 0; m < M; ++m)
    for (int64_t k = 0; k < K; ++k) xd[m * K + k] = r[m] * oracle_f16_to_f64(X[m * K + k]);
  int err = gemm_f64(W, xd, M, ncols, K, y, S);
  free(xd);
  return err;
}

/* SiLU of the SwiGLU feed-forward: v * sigmoid(v) = v / (1 + exp(-v)). */
void oracle_silu(const double* v, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = v[i] / (1.0 + exp(-v[i]));
}

/* ---- Q6_K, the other k-quant of Q4_K_M files --------------------------------
 * GGUF k-quant type Q6_K: a block of 256 weights in 210 bytes,
 *   ql[128]  the low 4 bits of the quants,
 *   qh[64]   the high 2 bits,
 *   sc[16]   int8 scales, one per run of 16 consecutive weights,
 *   d        binary16 super-scale (bytes 208-209, little-endian).
 * Weight k (0..255) lies in half h = k / 128, quarter j = (k % 128) / 32,
 * place l = k % 32. Its low bits are nibble j / 2 (0 low, 1 high) of
 * ql[64h + 32 (j % 2) + l], its high bits are bits 2j, 2j+1 of qh[32h + l];
 * q = low | high << 4 lies in 0..63 and w = d * sc[k / 16] * (q - 32). */
#define ORACLE_Q6K_BLOCK_BYTES 210

void oracle_q6k_dequant_block(const uint8_t* blk, double* w) {
  const double d = oracle_f16_to_f64((uint16_t)(blk[208] | (blk[209] << 8)));
  for (int k = 0; k < ORACLE_QK; ++k) {
    const int h = k / 128, j = (k % 128) / 32, l = k % 32;
    const int low = (blk[64 * h + 32 * (j % 2) + l] >> (4 * (j / 2))) & 15;
    const int high = (blk[128 + 32 * h + l] >> (2 * j)) & 3;
    const int q = low | (high << 4);
    w[k] = d * (double)(int8_t)blk[192 + k / 16] * (double)(q - 32);
  }
}

void oracle_q6k_dequant_row(const uint8_t* row, int64_t K, double* w) {
  for (int64_t b = 0; b < K / ORACLE_QK; ++b)
    oracle_q6k_dequant_block(row + b * ORACLE_Q6K_BLOCK_BYTES, w + b * ORACLE_QK);
}

void oracle_q6k_dequant_rows(const uint8_t* W, int64_t nrows, int64_t K, double* w) {
  for (int64_t n = 0; n < nrows; ++n)
    oracle_q6k_dequant_row(W + n * (K / ORACLE_QK) * ORACLE_Q6K_BLOCK_BYTES, K, w + n * K);
}

/* Reference GEMM over Q6_K rows: y = x * W^T, S = |x| * |W|^T, as oracle_gemm. */
int oracle_q6k_gemm(const uint8_t* W, const uint16_t* X, int64_t M, int64_t ncols, int64_t K,
                    double* y, double* S) {
  if (K % ORACLE_QK) return -1;
  double* xd = (double*)malloc(sizeof(double) * (size_t)(M * K));
  if (!xd) return -2;
  for (int64_t i = 0; i < M * K; ++i) xd[i] = oracle_f16_to_f64(X[i]);
  int err = gemm_f64_rows(W, K / ORACLE_QK * ORACLE_Q6K_BLOCK_BYTES, oracle_q6k_dequant_row, xd,
                          M, ncols, K, y, S);
  free(xd);
  return err;
}

/* Reference for a Q6_K matrix of the layer walk (a Q4_K_M file keeps v and
 * down in Q6_K in some layers): as oracle_gemm_std, the product of the
 * row-wise standardized binary16 input with the weights, here Q6_K rows
 * (oracle_q6k_dequant_block), everything in double. */
int oracle_q6k_gemm_std(const uint8_t* W, const uint16_t* X, int64_t M, int64_t ncols, int64_t K,
                        double eps, double* y, double* S) {
  if (K % ORACLE_QK) return -1;
  double* xd = (double*)malloc(sizeof(double) * (size_t)(M * K));
  double* t = (double*)malloc(sizeof(double) * (size_t)(M * K));
  if (!xd || !t) {
    free(xd);
    free(t);
    return -2;
  }
  for (int64_t i = 0; i < M * K; ++i) xd[i] = oracle_f16_to_f64(X[i]);
  oracle_standardize(xd, M, K, eps, t);
  int err = gemm_f64_rows(W, K / ORACLE_QK * ORACLE_Q6K_BLOCK_BYTES, oracle_q6k_dequant_row, t, M,
                          ncols, K, y, S);
  free(xd);
  free(t);
  return err;
}

/* ---- decode attention over a paged q8_0 KV pool ----------------------------
 * A page holds 16 tokens; page p, KV head h is 4352 bytes at (p*n_kv + h)*4352:
 * an int8 quant per K and V value and a binary16 scale per token and 32-dim
 * block b (dims 32b..32b+31 share it), a value being scale * quant (q8_0).
 * The 4096 quant bytes come first, as four 1 KiB slabs of 64 x 16 bytes, then
 * 64 bytes of scales per group of four tokens (K scales of tokens 4g..4g+3,
 * then their V scales, each [token][block]); the offset of every field is
 * written out in oracle_q8_page. */
#define ORACLE_PAGE_TOKENS 16
#define ORACLE_HEAD_DIM 128
#define ORACLE_PAGE_HEAD_BYTES 4352

/* K and V of one page-head as doubles, [16][128] each. */
void oracle_q8_page(const uint8_t* ph, double* k, double* v) {
  for (int t = 0; t < ORACLE_PAGE_TOKENS; ++t)
    for (int d = 0; d < ORACLE_HEAD_DIM; ++d) {
      const int b = d / 32;
      /* where the page-head keeps each field (the layout of the pool) */
      const int kq_at = 1024 * (b / 2) + 16 * (16 * ((d % 32) / 8) + t) + 8 * (b % 2) + d % 8;
      const int vq_at = 1024 * (2 + d / 64) + 16 * (16 * (t / 4) + d % 16) + 4 * ((d / 16) % 4) + t % 4;
      const int ks_at = 4096 + 64 * (t / 4) + 2 * (4 * (t % 4) + b);
      const int vs_at = ks_at + 32;
      const uint16_t ks = (uint16_t)(ph[ks_at] | (ph[ks_at + 1] << 8));
      const uint16_t vs = (uint16_t)(ph[vs_at] | (ph[vs_at + 1] << 8));
      k[t * ORACLE_HEAD_DIM + d] = oracle_f16_to_f64(ks) * (double)(int8_t)ph[kq_at];
      v[t * ORACLE_HEAD_DIM + d] = oracle_f16_to_f64(vs) * (double)(int8_t)ph[vq_at];
    }
}

/* The largest |V scale| of token t (0..15) of a page-head, over its four
 * 32-dim blocks (scales at the offsets oracle_q8_page reads them from). */
double oracle_q8_vscale_max(const uint8_t* ph, int t) {
  double mx = 0.0;
  for (int b = 0; b < 4; ++b) {
    const int vs_at = 4096 + 64 * (t / 4) + 2 * (4 * (t % 4) + b) + 32;
    const double v = fabs(oracle_f16_to_f64((uint16_t)(ph[vs_at] | (ph[vs_at + 1] << 8))));
    if (v > mx) mx = v;
  }
  return mx;
}

/* The floor of the attention error bound, in units of the largest V scale a
 * row attends to: 2^-80. A term p_i v_i[d] is held to fp32-like precision
 * only while its unnormalised weight times its V scale stays above about
 * fp32's smallest normal number, 2^-126, relative to twice that largest
 * scale; a term below that is at most 127 * 2^-125 = 2^-118 of it, and up to
 * 2^18 of them add at most 2^-100, less than the 2^-93.3 that 1e-4 times
 * 2^-80 allows. */
#define ORACLE_ATTN_FLOOR 0x1p-80

/* Reference decode attention. Row r of Q [M][n_heads][128] (binary16) belongs
 * to agent row_agent[r] and attends to that agent's first row_len[r] tokens,
 * token i living in page block_table[agent][i / 16], slot i % 16. Head h reads
 * KV head h / (n_heads / n_kv). In double precision:
 *   s_i = (q . k_i) / sqrt(128),  p = softmax(s),  O = sum_i p_i v_i,
 * and, for the error bound, per output element
 *   S[d] = sum_i p_i |v_i[d]| + 2^-80 * max_i |V scale of token i|,
 * the sum of the sizes of the terms O[d] adds, plus a floor at the edge of
 * fp32's range (ORACLE_ATTN_FLOOR). A row with no token to attend to
 * (row_len <= 0) gets O = 0 and S = 0: the empty sum. */
int oracle_q8_attn(const uint16_t* Q, const uint8_t* pool, const int32_t* block_table,
                   const int32_t* row_agent, const int32_t* row_len, int64_t M,
                   int64_t max_pages, int64_t n_heads, int64_t n_kv, double* O, double* S) {
  if (n_kv < 1 || n_heads % n_kv) return -1;
  const int64_t group = n_heads / n_kv;
  const double scale = 1.0 / sqrt((double)ORACLE_HEAD_DIM);
  int err = 0;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
  for (int64_t r = 0; r < M; ++r)
    for (int64_t h = 0; h < n_heads; ++h) {
      const int64_t n = row_len[r];
      const int64_t a = row_agent[r];
      const int64_t kvh = h / group;
      double* s = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
      double* k = (double*)malloc(sizeof(double) * ORACLE_PAGE_TOKENS * ORACLE_HEAD_DIM);
      double* v = (double*)malloc(sizeof(double) * ORACLE_PAGE_TOKENS * ORACLE_HEAD_DIM);
      double q[ORACLE_HEAD_DIM];
      double* o = O + (r * n_heads + h) * ORACLE_HEAD_DIM;
      double* sa = S + (r * n_heads + h) * ORACLE_HEAD_DIM;
      if (!s || !k || !v || n < 1) {
        if (n < 1) {  /* nothing to attend to: the empty weighted sum, 0 */
          for (int d = 0; d < ORACLE_HEAD_DIM; ++d) o[d] = sa[d] = 0.0;
        } else {
#pragma omp atomic write
          err = -2;
        }
        free(s);
        free(k);
        free(v);
        continue;
      }
      for (int d = 0; d < ORACLE_HEAD_DIM; ++d)
        q[d] = oracle_f16_to_f64(Q[(r * n_heads + h) * ORACLE_HEAD_DIM + d]);
      /* scores */
      double mx = -INFINITY;
      for (int64_t i = 0; i < n; ++i) {
        const int64_t page = block_table[a * max_pages + i / ORACLE_PAGE_TOKENS];
        if (i % ORACLE_PAGE_TOKENS == 0)
          oracle_q8_page(pool + (size_t)(page * n_kv + kvh) * ORACLE_PAGE_HEAD_BYTES, k, v);
        const double* ki = k + (i % ORACLE_PAGE_TOKENS) * ORACLE_HEAD_DIM;
        double dot = 0.0;
        for (int d = 0; d < ORACLE_HEAD_DIM; ++d) dot += q[d] * ki[d];
        s[i] = dot * scale;
        if (s[i] > mx) mx = s[i];
      }
      /* softmax weights and the weighted sum of values */
      double z = 0.0;
      for (int64_t i = 0; i < n; ++i) {
        s[i] = exp(s[i] - mx);
        z += s[i];
      }
      double vscale = 0.0;
      for (int d = 0; d < ORACLE_HEAD_DIM; ++d) o[d] = sa[d] = 0.0;
      for (int64_t i = 0; i < n; ++i) {
        const int64_t page = block_table[a * max_pages + i / ORACLE_PAGE_TOKENS];
        const uint8_t* ph = pool + (size_t)(page * n_kv + kvh) * ORACLE_PAGE_HEAD_BYTES;
        if (i % ORACLE_PAGE_TOKENS == 0) oracle_q8_page(ph, k, v);
        const double p = s[i] / z;
        const double* vi = v + (i % ORACLE_PAGE_TOKENS) * ORACLE_HEAD_DIM;
        for (int d = 0; d < ORACLE_HEAD_DIM; ++d) {
          o[d] += p * vi[d];
          sa[d] += p * fabs(vi[d]);
        }
        const double vs = oracle_q8_vscale_max(ph, (int)(i % ORACLE_PAGE_TOKENS));
        if (vs > vscale) vscale = vs;
      }
      for (int d = 0; d < ORACLE_HEAD_DIM; ++d) sa[d] += ORACLE_ATTN_FLOOR * vscale;
      free(s);
      free(k);
      free(v);
    }
  return err;
}

void oracle_f64_to_f16_array(const double* v, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_f64_to_f16(v[i]);
}

void oracle_f16_to_f64_array(const uint16_t* h, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_f16_to_f64(h[i]);
}

#ifdef _OPENMP
#include <omp.h>
#endif
/* Threads the oracle's parallel loops use. */
int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
