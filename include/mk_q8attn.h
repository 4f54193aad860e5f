/*
 * mk_q8attn.h - decode attention of stacked rows over a paged q8_0 KV pool
 * (part of libmkq4k.so; error codes are those of mk_q4k.h).
 *
 * The other growing cost of the multi-agent decode step (the OpenJet post,
 * "RTX 3090 one card, four coding agents", paragraph on how parallel
 * decoding works: once the weights are read once per step, what grows with
 * the agents is attention over their caches). n_agents agents each stack
 * rows_per_agent rows (next token + drafts): row r = a * rows_per_agent + j.
 *
 * KV pool (device, caller-owned): 16-token pages; page p, KV head h is 4352
 * bytes at (p * n_kv + h) * 4352. Token t's value in dim d is
 * scale(t, d / 32) * quant(t, d) (q8_0: one binary16 scale per 32 values,
 * int8 quants). Byte offsets within the page-head (b = d / 32):
 *   K quant (t, d)  1024 * (b / 2) + 16 * (16 * ((d % 32) / 8) + t)
 *                   + 8 * (b % 2) + d % 8
 *   V quant (t, d)  1024 * (2 + d / 64) + 16 * (16 * (t / 4) + d % 16)
 *                   + 4 * ((d / 16) % 4) + t % 4
 *   K scale (t, b)  4096 + 64 * (t / 4) + 2 * (4 * (t % 4) + b)
 *   V scale (t, b)  4096 + 64 * (t / 4) + 32 + 2 * (4 * (t % 4) + b)
 * That is, the 4096 quant bytes are four 1 KiB slabs of 64 x 16 bytes, the
 * 16 bytes at 16 * l of each slab being what lane l of a 64-wide wave feeds
 * to its matrix-core operands (slabs 0-1: K of token l % 16, slabs 2-3: V
 * of tokens 4 (l / 16) .. +3); the scales follow in 64-byte groups of four
 * tokens. A page then arrives as four fully contiguous 16-byte-per-lane
 * loads plus the scales, and neither product needs a transpose.
 *
 * Row r attends to the first row_len[r] tokens of its agent's sequence
 * (row_len <= 0: no token, and the row's output is 0, the empty sum);
 * token i of agent a lives in page block_table[a * max_pages + i / 16], slot
 * i % 16. Head h reads KV head h / (n_heads / n_kv). Head dimension 128.
 *   s_i = (q . k_i) / sqrt(128),   O = sum_i softmax(s)_i v_i
 * Precision: the int8 quants and binary16 queries enter the products
 * exactly; scores, softmax and sums in fp32; the weights times V scales go
 * to the value product as three bfloat16 parts that add up to each of them
 * exactly, down to fp32's normal range. Each output element is within
 * 1e-4 * (sum_i p_i |v_i[d]| + 2^-80 * V_max) of the exact result, V_max
 * the largest V scale the row attends to (the tests check this bound).
 * Deterministic, and each row's result does not depend on the other rows.
 */
#ifndef MK_Q8ATTN_H
#define MK_Q8ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Bytes of device workspace mk_q8_attn_decode needs (0 for invalid sizes). */
size_t mk_q8_attn_workspace_bytes(int n_agents, int max_pages, int n_kv);

/*
 * mk_q8_attn_decode: enqueue decode attention on `stream`.
 *   Q            device binary16 [M][n_heads][128], M = n_agents * rows_per_agent
 *   pool         device KV pool (layout above) of n_pages pages
 *   block_table  device int32 [n_agents][max_pages] page indices
 *   row_len      device int32 [M]; 1 <= row_len[r] <= 16 * (pages listed for its agent)
 *   O            device fp32 [M][n_heads][128], fully overwritten
 *   workspace    device, >= mk_q8_attn_workspace_bytes(n_agents, max_pages, n_kv),
 *                one call at a time
 * Requires n_kv >= 1, n_heads % n_kv == 0 and rows_per_agent * n_heads / n_kv
 * <= 32 (MK_EINVAL otherwise); Q, pool, O and workspace 16-byte aligned
 * (MK_EALIGN). Device arrays are not read on the host: the kernels clamp
 * lengths to 16 * max_pages and page indices into [0, n_pages), so values
 * outside the limits above give unspecified results but never an access
 * outside the pool.
 */
int mk_q8_attn_decode(const uint16_t* Q, const void* pool, int n_pages,
                      const int32_t* block_table, const int32_t* row_len, int n_agents,
                      int rows_per_agent, int max_pages, int n_heads, int n_kv, float* O,
                      void* workspace, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MK_Q8ATTN_H */
