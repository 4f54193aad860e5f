/*
 * mk_q4k.h - C ABI of the Q4_K weight-streaming decode GEMM for AMD MI355X
 * (gfx950).
 *
 * The operation (the OpenJet post, "RTX 3090 one card, four coding agents",
 * paragraph on how parallel decoding works): a decode step stacks the rows of
 * every active agent (next token plus two draft tokens each, 12 rows for four
 * agents) into one activation matrix X, streams every Q4_K weight of the model
 * from memory exactly once, and multiplies each weight, while it is on chip,
 * against all of the rows. The cost of a step is then about one weight read
 * however many rows ride along. The same paragraph states that the whole step
 * runs as one persistent kernel with no per-layer launches; mk_q4k_step is
 * that walk.
 *
 *   Y[m][n] = sum_k X[m][k] * w[n][k],   0 <= m < M, 0 <= n < N, 0 <= k < K
 *
 * Weights: Q4_K super-blocks of 256 weights in 144 bytes (the public GGUF
 * k-quant layout; the pages name the format "Q4_K_M"):
 *   bytes 0-1 d (binary16), 2-3 dmin (binary16), 4-15 packed 6-bit scales
 *   sc[8] and mins m[8], 16-143 4-bit quants q[256];
 *   w = d * sc[j] * q - dmin * m[j] for a weight of sub-block j (32 weights).
 * W holds N rows; row n is K/256 consecutive blocks, so block (n, kb) starts
 * at byte (n * (K/256) + kb) * 144. Subnormal d and dmin are honoured.
 *
 * Conventions for every call:
 *   - Pointers are DEVICE pointers owned by the caller unless marked (host).
 *     W, X and Y must be 16-byte aligned. Y must not overlap W or X.
 *   - stream is a hipStream_t passed as void* (NULL = the null stream).
 *   - Calls validate their arguments on the host (no device access), enqueue
 *     their kernels on `stream` and return; they do not synchronise and never
 *     print or abort. Errors are returned as negative codes.
 *   - Results are deterministic run to run (no floating-point atomics).
 *   - Accuracy. The kernels multiply the two terms of each weight apart,
 *     d * (sc[j] * q) against X and dmin * m[j] against X's 32-value
 *     sub-block sums, and subtract them in fp32 (every product exact, only
 *     fp32 sums rounded). Each output element is within 1e-4 * F[m][n] of
 *     the exact result, F[m][n] = sum_k (|d sc[j] q[k]| + |dmin m[j]|) *
 *     |X[m][k]|, for any finite binary16 X. Where a weight's two terms do not
 *     nearly cancel, F is a small multiple of S[m][n] = sum_k |w[n][k] *
 *     X[m][k]| and the error is within 1e-4 * S: this holds for the
 *     workload's generated weights and is what the tests check there. Blocks
 *     whose weights are (nearly) zero because the two terms cancel (d*sc*q
 *     close to dmin*m over a whole sub-block) get the F bound only: an
 *     exactly cancelling block gives a tiny nonzero result, not an exact 0.
 *     An output is exactly 0 where F is 0.
 */
#ifndef MK_Q4K_H
#define MK_Q4K_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
#define MK_OK 0
#define MK_EINVAL (-1)     /* bad shape, null pointer or broken layer chain   */
#define MK_EALIGN (-2)     /* W, X, Y (or a step buffer) not 16-byte aligned  */
#define MK_EWORKSPACE (-3) /* workspace missing or smaller than required      */
#define MK_EOCCUPANCY (-4) /* the persistent grid cannot be co-resident       */
#define MK_EHIP (-5)       /* a HIP runtime call failed (see mk_strerror)     */
#define MK_ENODEV (-6)     /* the current device is not a gfx950 GPU          */
#define MK_ETIMEOUT (-7)   /* device status: a cross-workgroup wait timed out  */
#define MK_ERANGE (-8)     /* device status: a row statistic left its range    */

#define MK_Q4K_QK 256          /* weights per super-block                   */
#define MK_Q4K_BLOCK_BYTES 144 /* bytes per super-block                     */
#define MK_Q4K_MAX_M 64        /* most stacked rows one call accepts        */

/*
 * mk_q4k_gemm: Y = X * W^T for one Q4_K matrix.
 *   W_blocks  N * (K/256) blocks of 144 bytes, layout above.
 *   X_fp16    [M][K] binary16, row-major, row stride K.
 *   Y_fp32    [M][N] float, row-major, row stride N; fully overwritten.
 *   M         1..64 stacked rows; N >= 1; K >= 256 and K % 256 == 0.
 * One launch of one workgroup per compute unit; when K is cut into several
 * slices, the slice partial sums go to a device workspace and a second
 * kernel, enqueued on the same stream, adds them in slice order.
 * Batch invariance: the K slices are chosen for MK_Q4K_MAX_M rows whatever
 * M is, so each output is summed in an order that depends on N, K and the
 * device only: a row of Y is the same, bit for bit, whether X holds it alone
 * or stacked with any other rows (the same holds for mk_q4k_gemm_tiled, and
 * the two agree bit for bit).
 * Returns MK_OK or MK_EINVAL / MK_EALIGN / MK_ENODEV / MK_EHIP. The library
 * keeps a private device workspace per (GPU, stream) for the K-split partial
 * sums: the first call on a stream that needs more than that stream's
 * workspace holds allocates a larger one (hipMalloc; it never synchronises,
 * and a smaller one it replaces stays allocated, since queued work may still
 * read it, until the process ends); later calls allocate nothing. Calls on
 * one stream are ordered by the stream; a caller that cannot allocate uses
 * mk_q4k_gemm_ws.
 */
int mk_q4k_gemm(const void* W_blocks, const uint16_t* X_fp16, float* Y_fp32, int M, int N, int K,
                void* stream);

/*
 * mk_q4k_gemm_ws: as mk_q4k_gemm with a caller-provided workspace of at least
 * mk_q4k_gemm_workspace_bytes(M, N, K) bytes (16-byte aligned device memory,
 * used by one call at a time; its contents need no initialisation and are
 * overwritten by every call). It never allocates. The size depends on the current device's compute-unit count
 * (256 is assumed when there is none). A shape whose slice partials would
 * take 4 GiB or more returns MK_EINVAL.
 */
size_t mk_q4k_gemm_workspace_bytes(int M, int N, int K);
int mk_q4k_gemm_ws(const void* W_blocks, const uint16_t* X_fp16, float* Y_fp32, int M, int N,
                   int K, void* workspace, size_t ws_bytes, void* stream);

/*
 * mk_q4k_gemm_noalloc: mk_q4k_gemm for callers that cannot allocate (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc). Same arguments, kernels and results (bit for bit) as
 * mk_q4k_gemm; it calls no hipMalloc, hipFree or other allocating routine.
 * The K-split partial sums go to a device array of
 * MK_Q4K_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs
 * on until the process ends (enough for every shape of the 27B-class layer
 * up to 64 rows). A shape whose partials need more returns MK_EWORKSPACE
 * before anything is enqueued (use mk_q4k_gemm_ws for it). The first call on
 * a device looks up that device's copy of the array (hipGetSymbolAddress).
 * All calls on one GPU share the array: calls that overlap in time on one
 * GPU (different streams, not ordered) race and give wrong results. Its
 * contents need no initialisation; each call overwrites what it reads.
 */
#define MK_Q4K_NOALLOC_SCRATCH_BYTES (24 << 20)
int mk_q4k_gemm_noalloc(const void* W_blocks, const uint16_t* X_fp16, float* Y_fp32, int M, int N,
                        int K, void* stream);

/*
 * Tile records: a load-time reordering of a Q4_K matrix for the streaming
 * kernels. Every block keeps its 144 bytes; rows are grouped in tiles of 16
 * (rows past N are zero blocks) and for tile t and super-block kb the
 * 2304-byte record at (t * (K/256) + kb) * 2304 holds the 16 block headers
 * (bytes 0-15 of each block, row order), then for l = 0..63 (row i = l % 16,
 * g = l / 16) quant bytes [32g, 32g+16) of row i, then for the same l quant
 * bytes [32g+16, 32g+32). A wave then reads each operand with one contiguous
 * 1 KiB load instead of sixteen 16-byte pieces 2.9 KB apart.
 *
 * The records are followed by ceil(N/16)*16 fp32 column sums: entry n is
 * sum_k w[n][k] over the exact dequantized weights of row n (0 for padding
 * rows), rounded once to fp32. The decode-step walk uses them to apply the
 * row standardization of its inputs after the product (see mk_q4k_step).
 *
 * mk_q4k_tiles_bytes: size of the record form of an N x K matrix
 *   (ceil(N/16) * ((K/256) * 2304 + 64)), 0 for an invalid shape.
 * mk_q4k_repack: write the record form of W_rows (layout above, N rows) to
 *   W_tiles (device, mk_q4k_tiles_bytes bytes, must not overlap W_rows).
 *   Asynchronous on `stream`; MK_OK, MK_EINVAL, MK_EALIGN or MK_EHIP.
 */
size_t mk_q4k_tiles_bytes(int N, int K);
int mk_q4k_repack(const void* W_rows, void* W_tiles, int N, int K, void* stream);

/*
 * mk_q4k_gemm_tiled: mk_q4k_gemm on the tile-record form of W (W_tiles, made
 * once by mk_q4k_repack at load time). Same arguments, results (bit for bit:
 * the same kernel and arithmetic order), errors and workspace behaviour; the
 * weight stream reads whole 1 KiB pieces instead of 16-byte pieces of 16
 * rows.
 */
int mk_q4k_gemm_tiled(const void* W_tiles, const uint16_t* X_fp16, float* Y_fp32, int M, int N,
                      int K, void* stream);

/*
 * The decode-step walk: one persistent kernel launch runs n_layers layers of
 * seven Q4_K matrices each, in their data-dependency order. No grid-wide
 * barrier is used: a phase's outputs are counted into device counters and the
 * next phase starts on every workgroup as soon as those counters show that its
 * whole input exists:
 *   phase A  x_l                -> q [M, Nq], k [M, Nk], v [M, Nv]
 *   phase B  c(q)               -> o [M, H]
 *   phase C  c(o)               -> gate [M, F], up [M, F]
 *   phase D  c(gate * up)       -> down [M, H]     (product elementwise, fp32)
 *   x_{l+1} = c(down)
 * where c is the binary16 round-to-nearest-even cast (the workload's "fp32 to
 * fp16 cast" between layers). Every matrix multiplies the row-standardized
 * form of its binary16 input x:
 *   y[m][n] = sum_k (x[m][k] - mean_m) / sqrt(var_m + 1e-6) * w[n][k],
 * mean and population variance over the K values of row m of x, applied
 * exactly (never rounded to binary16): the kernel computes
 * (sum_k x*w - mean_m * colsum_n) / sqrt(var_m + 1e-6) with the column sums
 * mk_q4k_repack stores after the records. Without the standardization the
 * chained products leave the binary16 range within one layer. The layer input
 * x_0 is given; every later input is produced on the device. k and v are
 * written but feed nothing (in a model they would feed attention, which is
 * not part of this walk).
 *
 * Accuracy: each output is within 1e-4 * r_m * (F + |mean_m * colsum_n|) of
 * the product with the exactly standardized input, F as above over the
 * binary16 input x and r_m = 1 / sqrt(var_m + 1e-6); for the workload's
 * weights and N(0,1) inputs that is within 1e-4 * sum_k |w[n][k] * t[m][k]|,
 * t the standardized input (what the tests check on every matrix).
 *
 * Batch invariance: every phase's K slices are chosen for 16 rows whatever
 * M is, and a row's statistics are exact integer sums of its own values, so
 * each row's outputs and phase inputs are the same, bit for bit, whether it
 * is walked alone or stacked with other rows (mk_q4k_step_res likewise).
 *
 * Rows past 16 (a prefill chunk riding with the decode rows; the OpenJet
 * post, paragraph on keeping it fast with real agents): one walk takes one
 * MFMA row tile of 16 rows, so a call with M > 16 runs ceil(M / 16) walks one
 * after another on the stream, rows [16g, 16g + 16) in walk g, each streaming
 * every weight once. By the invariance above a row's results do not depend
 * on its group. The workspace of 16 rows serves every M; the status word
 * keeps the first failure of any group.
 *
 * Chain rules (checked): q.K = k.K = v.K = gate.K = up.K = down.N = H (the
 * hidden size), o.K = q.N, gate.N = up.N = down.K = F; every K % 256 == 0;
 * every layer has the same shapes. Limits: 1 <= M <= 64 stacked rows,
 * 1 <= n_layers <= 128, each matrix's tile-record form under 4 GiB
 * (otherwise MK_EINVAL). Each phase's K range is cut into slices whose input
 * rows fit in on-chip memory; a shape whose plan still does not fit one
 * workgroup per compute unit returns MK_EOCCUPANCY.
 */
/* Block types of a step matrix (GGUF type numbers); 0 means Q4_K. */
#define MK_QTYPE_Q4_K 12
#define MK_QTYPE_Q6_K 14

typedef struct {
  const void* w; /* device: the record form of the matrix: mk_q4k_repack for
                    Q4_K, mk_q6k_step_repack (mk_q6k.h) for Q6_K */
  int N;         /* output columns (weight rows)    */
  int K;         /* input width                     */
  int type;      /* MK_QTYPE_Q4_K (or 0) or MK_QTYPE_Q6_K; Q6_K only for v and
                    down, the matrices a Q4_K_M file keeps in Q6_K (else
                    MK_EINVAL); it may differ from layer to layer */
} mk_q4k_mat;

typedef struct {
  mk_q4k_mat q, k, v, o, gate, up, down;
} mk_q4k_layer;

/* Per-layer outputs the step writes (device pointers, caller-owned). */
typedef struct {
  float* y[7];    /* fp32 [M][N_t] for t = q, k, v, o, gate, up, down          */
  uint16_t* x[4]; /* binary16 phase inputs A..D: x_l [M][H], c(q) [M][q.N],
                     c(o) [M][H], c(gate*up) [M][F]                            */
} mk_q4k_layer_io;

/* Bytes of device workspace mk_q4k_step needs for this shape. */
size_t mk_q4k_step_workspace_bytes(const mk_q4k_layer* layer0 /* host */, int n_layers, int M);

/*
 * mk_q4k_step: run the walk.
 *   layers    (host) n_layers layer descriptors, read before return.
 *   io        (host) n_layers output descriptors, read before return.
 *   x0        [M][H] binary16 input of layer 0.
 *   x_out     [M][H] binary16 c(down) of the last layer.
 *   workspace device memory of >= mk_q4k_step_workspace_bytes bytes, used by
 *             one call at a time (calls that overlap on one workspace race);
 *             it holds the phase counters, the device status word, row
 *             statistics, partial sums and the copied descriptor tables.
 *             The call clears what must start at zero itself.
 * Returns MK_OK (enqueued) or a host-side error. Device-side failures (a
 * counter wait that times out, a statistic out of range) are recorded in the
 * workspace status word; read it with mk_q4k_step_status after the stream
 * has been synchronised. MK_ERANGE there means a cast overflowed binary16 or
 * a row sum left the fixed-point range of the statistics (a term of 2^50).
 */
int mk_q4k_step(const mk_q4k_layer* layers, const mk_q4k_layer_io* io, int n_layers, int M,
                const uint16_t* x0, uint16_t* x_out, void* workspace, size_t ws_bytes,
                void* stream);

/*
 * The residual walk: the same persistent kernel and products, with the
 * epilogues of a real decoder layer around them in place of the
 * standardization (the OpenJet post, "RTX 3090 one card, four coding
 * agents", paragraph on how parallel decoding works: the one-kernel step
 * includes the work on either side of each product). With h the fp32
 * residual stream entering layer l and g_attn, g_ffn its fp32 RMSNorm
 * weights [H]:
 *   phase A  x_l = c(h * g_attn)        -> q, k, v = r(h) * (x_l . W)
 *   phase B  c(q)                       -> o;    h_mid = h + o
 *   phase C  c(h_mid * g_ffn)           -> gate, up = r(h_mid) * (x . W)
 *   phase D  c(silu(gate) * up)         -> down; h_out = h_mid + down
 * where c is the binary16 round-to-nearest-even cast of the fp32 value
 * (products, sums and silu(v) = v / (1 + exp(-v)) in fp32), and
 * r(h) = 1 / sqrt(mean_k h^2 + 1e-6) per row, applied exactly after the
 * product (so the cast is of h * g, not of the normalised value). The
 * attention between B and o is not part of the walk: o multiplies c(q).
 * h_out of layer l is the residual entering layer l + 1; h0 enters layer 0.
 * Shapes, limits, the workspace (mk_q4k_step_workspace_bytes) and the
 * status word are those of mk_q4k_step; MK_ERANGE there also means a cast
 * overflowed binary16 or a row's sum of squares left its range (a tile
 * row's sum of h^2 of 2^42).
 */
typedef struct {
  float* y[7];    /* fp32 [M][N_t] for t = q, k, v, o, gate, up, down          */
  uint16_t* x[4]; /* binary16 phase inputs A..D: c(h*g_attn) [M][H], c(q) [M][q.N],
                     c(h_mid*g_ffn) [M][H], c(silu(gate)*up) [M][F]            */
  float* h_mid;   /* fp32 [M][H] residual after o                              */
  float* h_out;   /* fp32 [M][H] residual after down                           */
} mk_q4k_layer_res_io;

typedef struct {
  const float* attn; /* fp32 [H] RMSNorm weight of the q/k/v input (device)      */
  const float* ffn;  /* fp32 [H] RMSNorm weight of the gate/up input (device)    */
} mk_q4k_layer_norm;

/*
 * mk_q4k_step_res: run the residual walk. layers, norms and io are host
 * arrays of n_layers entries, read before return; h0 is the device fp32
 * [M][H] residual entering layer 0. Every device pointer is 16-byte aligned
 * (MK_EALIGN otherwise); the output buffers must not overlap one another or
 * the inputs.
 */
int mk_q4k_step_res(const mk_q4k_layer* layers, const mk_q4k_layer_norm* norms,
                    const mk_q4k_layer_res_io* io, int n_layers, int M, const float* h0,
                    void* workspace, size_t ws_bytes, void* stream);

/*
 * mk_q4k_step_check_plan: host-only self-check of the walk's work split (no
 * device access). Plans the walk for layer0's shapes, n_layers layers, M rows
 * and G workgroups, walks every access the kernel's index arithmetic makes
 * (weight records, column sums, slice partials, LDS slots, staged rows,
 * finishing tiles, statistics slots) and returns how many fall outside their
 * buffer, or which tile is finished or covered other than once (0: none);
 * MK_EINVAL for invalid shapes, -1 when no plan fits (mk_q4k_step then
 * returns MK_EINVAL without launching).
 */
long long mk_q4k_step_check_plan(const mk_q4k_layer* layer0 /* host */, int n_layers, int M,
                                 int G);

/*
 * mk_q4k_step_set_walk_form: a testing aid that selects other forms of the
 * walks, which compute the same results bit for bit. Flags, OR-ed:
 * MK_WALK_AUTO (0, the default): a wave reads its records' addresses from a
 * per-phase record table held in registers (a branch-free streaming loop)
 * whenever every wave of every phase has at most 64 records, else it walks
 * them with the record iterator; a phase reloads the row statistics of its
 * input at the end of its compute only if some workgroup's share was not yet
 * added when it staged them.
 * MK_WALK_ITERATOR: always the record iterator.
 * MK_WALK_RELOAD_STATS: every phase reloads its input statistics (the path
 * otherwise taken only when a share arrives late).
 * Process-wide; applies to step calls made after it returns (a call already
 * enqueued keeps its form). MK_EINVAL for any other bit.
 */
#define MK_WALK_AUTO 0
#define MK_WALK_ITERATOR 1
#define MK_WALK_RELOAD_STATS 2
int mk_q4k_step_set_walk_form(int form);

/*
 * mk_q4k_step_timeline_offset: a measurement aid. In a library built with
 * MK_STEP_TIMELINE=1 the walks store, per layer l, phase p (0..3) and
 * workgroup w (G = the device's CU count), eight u64 wall-clock slots
 * (100 MHz) at byte offset + ((l * 4 + p) * G + w) * 64 of the workspace:
 * [0] input staged (compute starts), [1] compute ends, [2] slice partials
 * published, [3] own tiles finished, [4] the phase's done counters seen.
 * Returns that offset, or -1 in the product library (built without it).
 */
long long mk_q4k_step_timeline_offset(const mk_q4k_layer* layer0 /* host */, int n_layers, int M);

/* Copy the device status word of the last step run in `workspace` to
 * *status_out (MK_OK, MK_ETIMEOUT or MK_ERANGE). Synchronous; call after the
 * step's stream has completed. */
int mk_q4k_step_status(const void* workspace, int* status_out);

/*
 * mk_hbm_read_probe: a measurement, not part of the product path (the read
 * ceiling the weight stream is compared with). Reads every whole 16-byte word of
 * buf[0, bytes) once with nontemporal loads: `grid` workgroups of 512
 * threads, each streaming one contiguous share with eight loads in flight
 * per thread, and writes the XOR of what workgroup g read to out[g] (device,
 * grid words). buf 16-byte aligned (MK_EALIGN); bytes >= 16 and
 * 1 <= grid <= 65535 (MK_EINVAL). Asynchronous on `stream`.
 */
int mk_hbm_read_probe(const void* buf, size_t bytes, uint32_t* out, int grid, void* stream);

/* Static text for a return code (never NULL). */
const char* mk_strerror(int code);

/* Describe the current device (name, arch, CU count, LDS per block, clock)
 * into buf; returns MK_OK or MK_ENODEV / MK_EINVAL. */
int mk_device_info(char* buf, size_t len);

#ifdef __cplusplus
}
#endif

#endif /* MK_Q4K_H */
