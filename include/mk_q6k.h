/*
 * mk_q6k.h - Q6_K weights times stacked binary16 rows (part of
 * libmkq4k.so; error codes are those of mk_q4k.h).
 *
 * Q4_K_M model files (the format the OpenJet post's engine streams, "RTX
 * 3090 one card, four coding agents") are mostly Q4_K with some tensors in
 * Q6_K, the GGUF k-quant of 6 bits per weight: a block of 256 weights in
 * 210 bytes,
 *   bytes   0..127  ql: low 4 bits of the quants
 *   bytes 128..191  qh: high 2 bits of the quants
 *   bytes 192..207  sc: int8 scale of each run of 16 consecutive weights
 *   bytes 208..209  d: binary16 super-scale, little-endian
 * Weight k of a block (half h = k / 128, quarter j = (k % 128) / 32, place
 * l = k % 32) has low bits nibble j / 2 (0: low) of ql[64h + 32 (j % 2) + l]
 * and high bits 2j..2j+1 of qh[32h + l]; with q = low | high << 4 (0..63)
 * its value is d * sc[k / 16] * (q - 32). A weight row of K values (K a
 * multiple of 256) is K / 256 consecutive blocks.
 *
 * As for Q4_K, the weights are repacked once at load time into tile records
 * of 16 rows x one block (3360 bytes, laid out for the matrix-core lanes),
 * and the product streams those records once per call.
 *
 * Precision: the quants enter the matrix cores as exact binary16 q - 32,
 * the activations as given; each run of 16 products is summed in fp32 and
 * scaled by d * sc in fp32. Deterministic (fixed summation order for given
 * N and K, whatever M).
 */
#ifndef MK_Q6K_H
#define MK_Q6K_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MK_Q6K_BLOCK_BYTES 210 /* bytes per block of 256 weights */
#define MK_Q6K_TILE_BYTES 3360 /* bytes per tile record: 16 rows x one block */

/* Bytes of the tile-record form of an N x K Q6_K matrix: ceil(N / 16) *
 * (K / 256) * 3360. 0 if N < 1 or K is not a positive multiple of 256. */
size_t mk_q6k_tiles_bytes(int N, int K);

/* Repack W (device, N rows x K/256 blocks of 210 bytes, row-major, any
 * alignment) into `tiles` (device, caller-owned, mk_q6k_tiles_bytes(N, K)
 * bytes, 16-byte aligned); rows past N are zero. Asynchronous on `stream`
 * (a hipStream_t; NULL = the null stream). Returns MK_OK, MK_EINVAL (null
 * pointer or bad shape), MK_EALIGN or MK_EHIP. */
int mk_q6k_repack(const void* W, void* tiles, int N, int K, void* stream);

/* Y = X * W^T for the repacked Q6_K matrix W (N x K): X binary16 [M][K]
 * row-major, Y fp32 [M][N] row-major (device, caller-owned, 16-byte
 * aligned), 1 <= M <= 64. One launch takes up to 32 rows (two MFMA row
 * tiles); rows 32.. go to a second launch over the same weights on the same
 * stream. A row's result does not depend on the rows beside it, so every
 * row's bits are the same alone or stacked. Asynchronous on `stream`; no
 * workspace. Returns MK_OK, MK_EINVAL, MK_EALIGN or MK_EHIP. */
int mk_q6k_gemm_tiled(const void* tiles, const uint16_t* X, float* Y, int M, int N, int K,
                      void* stream);

/*
 * Q6_K matrices inside the decode-step walk (mk_q4k_step): a Q4_K_M file
 * keeps attn_v and ffn_down (in some or all layers) in Q6_K, and the walk
 * takes them as they are, in one launch with the Q4_K matrices (the OpenJet
 * post, paragraph on how parallel decoding works: the whole step in one
 * persistent kernel).
 *
 * mk_q6k_step_bytes: size of the walk's record form of an N x K Q6_K matrix
 *   (0 for a bad shape): ceil(N/16) * K/256 records of 3360 bytes, then
 *   ceil(N/16) * 16 fp32 column sums.
 * mk_q6k_step_repack: write that form of W (device, N rows x K/256 blocks of
 *   210 bytes, row-major, any alignment) to `out` (device, caller-owned,
 *   mk_q6k_step_bytes bytes, 16-byte aligned, not overlapping W). Each
 *   record holds 16 rows x one block in the lane order of the walk's
 *   activation operands (every byte of the block kept, reordered; rows past N
 *   zero); the column sums are sum_k w[n][k], exact per block in double,
 *   rounded once to fp32. Asynchronous on `stream`. Returns MK_OK, MK_EINVAL
 *   (null pointer, bad shape, overlap), MK_EALIGN or MK_EHIP.
 * Pass the result as the `w` of a layer's v or down matrix with type
 * MK_QTYPE_Q6_K (mk_q4k.h).
 */
size_t mk_q6k_step_bytes(int N, int K);
int mk_q6k_step_repack(const void* W, void* out, int N, int K, void* stream);

/* Y = X * W^T for a Q6_K matrix W (N x K) in the walk's record form above
 * (the column sums after the records are not read): X binary16 [M][K]
 * row-major, Y fp32 [M][N] row-major (device, caller-owned, 16-byte aligned,
 * Y overlapping neither), 1 <= M <= 64. The persistent product of
 * mk_q4k_gemm_tiled (mk_q4k.h) on Q6_K records: one workgroup per compute
 * unit, the K range cut into slices chosen from N, K and the device only
 * (not M), every record read once per call and multiplied against all M
 * rows (up to four 16-row MFMA tiles) while it is on chip, a second launch
 * adding each tile's slice partials in slice order when there are several;
 * so a row's bits are the same alone or stacked. The arithmetic is the
 * walk's: each operand d-free s * (q - 32) enters the matrix cores exactly,
 * as binary16 hi + lo, and each record's products are scaled by d in fp32.
 * The slice partials go to a library-owned workspace, as for mk_q4k_gemm.
 * Asynchronous on `stream`. Returns MK_OK, MK_EINVAL, MK_EALIGN, MK_ENODEV
 * or MK_EHIP. */
int mk_q6k_gemm_step(const void* W_step, const uint16_t* X, float* Y, int M, int N, int K,
                     void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MK_Q6K_H */
