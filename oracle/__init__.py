"""CPU oracle for the Q4_K weight-streaming decode GEMM - TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. The product path (the HIP library and
its binding) never does, and the two share no code: the arithmetic here lives
in ``q4k_oracle.c`` (plain C, double precision, compiled with gcc) and in the
few numpy lines below that only marshal arrays.

What it computes, and where that comes from:

* ``gemm``: ``y[m,n] = sum_k x[m,k] w[n,k]`` and ``S[m,n] = sum_k |x w|`` with
  w the exact dequantized Q4_K weight (the OpenJet post, "RTX 3090 one card,
  four coding agents", paragraph on how parallel decoding works: the stacked
  rows all multiply the same weights, read once). Pinned by the hand-built
  blocks, the constant-scale closed form and the numpy cross-checks in
  ``tests/test_oracle_pins.py``.
* ``decode_block`` / ``dequant_rows``: the Q4_K block (public GGUF layout;
  the pages name only "Q4_K_M"). Pinned by hand-built bytes, single-nibble
  unit vectors and exhaustive scale/min round trips.
* ``standardize`` / ``gemm_std``: every matrix of the layer walk multiplies
  the row-wise standardized form (mean 0, variance 1 per row, exact in
  float64) of its binary16 input; the phase inputs themselves are plain
  binary16 casts of the previous outputs. Pinned by closed-form moments, by
  invariance of ``gemm_std`` to a per-row shift and power-of-two scale of the
  input, by constant rows (output exactly 0) and by a numpy cross-check.
  ``f64_to_f16`` is pinned to numpy's binary16 cast.
* ``rms_inv`` / ``gemm_rms`` / ``silu``: the residual walk (real-layer
  epilogues around the same products): each normed matrix multiplies the
  binary16 cast of the residual times the norm weight, scaled per row by
  1 / sqrt(mean(h^2) + eps) of the fp32 residual h; the feed-forward input
  is SiLU(gate) * up. Pinned by constant rows, exact power-of-two scaling,
  the reduction of ``gemm_rms`` to ``gemm`` at unit scale, the SiLU
  identity silu(v) - silu(-v) = v and its limits, and numpy cross-checks.
* ``q8_page`` / ``attn_decode``: decode attention of stacked rows over a
  paged q8_0 KV pool (each row attends to its agent's first row_len tokens;
  softmax of q.k / sqrt(128), weighted sum of v), in float64; its bound S is,
  per output element, sum_i p_i |v_i[d]| plus a floor of 2^-80 times the
  largest V scale the row attends to (the edge of fp32's range). Pinned by
  hand-built pages, a single token (O = v), equal keys (O = mean v), two
  tokens in closed form, shift invariance of the scores and a numpy
  cross-check.
* ``factored_size`` / ``row_moments``: the size of the two terms of the
  factored weight, sum_k (|d sc q| + |dmin m|) |x|, against which a product
  that applies d and dmin separately keeps its error where the terms nearly
  cancel (plus |mean * colsum| and the row scale for a matrix of the walk).
  Pinned by a hand-worked block, by F == S where no weight's terms have
  opposite signs, and by F >= S everywhere.
* ``within_bound``: the acceptance rule ``|y - y_ref| <= tol * S``, and
  ``y == 0`` exactly where ``S == 0``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

BLOCK_BYTES = 144
QK = 256
TOL = 1e-4


def build(force: bool = True) -> str:
    """Compile liboracle.so in place (gcc -O2, strict C11: no fp contraction,
    no fast-math)."""
    src = os.path.join(_HERE, "q4k_oracle.c")
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", src, "-o", tmp, "-lm"]
        )
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        lib = ctypes.CDLL(_LIB_PATH)
        vp = ctypes.c_void_p
        i64 = ctypes.c_int64
        lib.oracle_f16_to_f64.restype = ctypes.c_double
        lib.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
        lib.oracle_f64_to_f16.restype = ctypes.c_uint16
        lib.oracle_f64_to_f16.argtypes = [ctypes.c_double]
        lib.oracle_f16_to_f64_array.restype = None
        lib.oracle_f16_to_f64_array.argtypes = [vp, i64, vp]
        lib.oracle_f64_to_f16_array.restype = None
        lib.oracle_f64_to_f16_array.argtypes = [vp, i64, vp]
        lib.oracle_unpack_scales.restype = None
        lib.oracle_unpack_scales.argtypes = [vp, vp, vp]
        lib.oracle_decode_block.restype = None
        lib.oracle_decode_block.argtypes = [vp, vp, vp, vp, vp, vp]
        lib.oracle_dequant_rows.restype = None
        lib.oracle_dequant_rows.argtypes = [vp, i64, i64, vp]
        lib.oracle_gemm.restype = ctypes.c_int
        lib.oracle_gemm.argtypes = [vp, vp, i64, i64, i64, vp, vp]
        lib.oracle_q6k_dequant_rows.restype = None
        lib.oracle_q6k_dequant_rows.argtypes = [vp, i64, i64, vp]
        lib.oracle_q6k_gemm.restype = ctypes.c_int
        lib.oracle_q6k_gemm.argtypes = [vp, vp, i64, i64, i64, vp, vp]
        lib.oracle_gemm_std.restype = ctypes.c_int
        lib.oracle_gemm_std.argtypes = [vp, vp, i64, i64, i64, ctypes.c_double, vp, vp]
        lib.oracle_q6k_gemm_std.restype = ctypes.c_int
        lib.oracle_q6k_gemm_std.argtypes = [vp, vp, i64, i64, i64, ctypes.c_double, vp, vp]
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_num_threads.argtypes = []
        lib.oracle_standardize.restype = None
        lib.oracle_standardize.argtypes = [vp, i64, i64, ctypes.c_double, vp]
        lib.oracle_row_moments.restype = None
        lib.oracle_row_moments.argtypes = [vp, i64, i64, ctypes.c_double, vp, vp]
        lib.oracle_factored_size.restype = ctypes.c_int
        lib.oracle_factored_size.argtypes = [vp, vp, i64, i64, i64, vp, vp, vp]
        lib.oracle_rms_inv.restype = None
        lib.oracle_rms_inv.argtypes = [vp, i64, i64, ctypes.c_double, vp]
        lib.oracle_gemm_rms.restype = ctypes.c_int
        lib.oracle_gemm_rms.argtypes = [vp, vp, i64, i64, i64, vp, vp, vp]
        lib.oracle_q8_vscale_max.restype = ctypes.c_double
        lib.oracle_q8_vscale_max.argtypes = [vp, ctypes.c_int]
        lib.oracle_q8_page.restype = None
        lib.oracle_q8_page.argtypes = [vp, vp, vp]
        lib.oracle_q8_attn.restype = ctypes.c_int
        lib.oracle_q8_attn.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, vp, vp]
        lib.oracle_silu.restype = None
        lib.oracle_silu.argtypes = [vp, i64, vp]
        _lib = lib
    return _lib


def _c(a: np.ndarray, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


def f16_to_f64(bits) -> np.ndarray:
    """Decode binary16 bit patterns (uint16 array, or float16 array) to float64."""
    h = np.asarray(bits)
    if h.dtype == np.float16:
        h = h.view(np.uint16)
    h = _c(h, np.uint16)
    out = np.empty(h.shape, dtype=np.float64)
    _load().oracle_f16_to_f64_array(h.ctypes.data, h.size, out.ctypes.data)
    return out


def f64_to_f16(v) -> np.ndarray:
    """Round float64 values to binary16 (nearest, ties to even); returns uint16 bits."""
    v = _c(v, np.float64)
    out = np.empty(v.shape, dtype=np.uint16)
    _load().oracle_f64_to_f16_array(v.ctypes.data, v.size, out.ctypes.data)
    return out


def unpack_scales(s12) -> tuple[np.ndarray, np.ndarray]:
    s = _c(np.frombuffer(bytes(s12), dtype=np.uint8), np.uint8)
    if s.size != 12:
        raise ValueError("need 12 bytes")
    sc = np.zeros(8, dtype=np.int32)
    mn = np.zeros(8, dtype=np.int32)
    _load().oracle_unpack_scales(s.ctypes.data, sc.ctypes.data, mn.ctypes.data)
    return sc, mn


def decode_block(blk) -> tuple[float, float, np.ndarray, np.ndarray, np.ndarray]:
    b = _c(np.frombuffer(bytes(blk), dtype=np.uint8), np.uint8)
    if b.size != BLOCK_BYTES:
        raise ValueError("a Q4_K block is 144 bytes")
    d = np.zeros(1, dtype=np.float64)
    dmin = np.zeros(1, dtype=np.float64)
    sc = np.zeros(8, dtype=np.int32)
    mn = np.zeros(8, dtype=np.int32)
    q = np.zeros(256, dtype=np.int32)
    _load().oracle_decode_block(b.ctypes.data, d.ctypes.data, dmin.ctypes.data, sc.ctypes.data,
                                mn.ctypes.data, q.ctypes.data)
    return float(d[0]), float(dmin[0]), sc, mn, q


def dequant_rows(W: np.ndarray, K: int) -> np.ndarray:
    """Exact float64 weights [nrows, K] of Q4_K rows W (uint8 [nrows, K/256*144])."""
    W = _c(W, np.uint8)
    nrows = W.size // (K // QK * BLOCK_BYTES)
    out = np.empty((nrows, K), dtype=np.float64)
    _load().oracle_dequant_rows(W.ctypes.data, nrows, K, out.ctypes.data)
    return out


def gemm(W: np.ndarray, X: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Reference (y, S), both float64 [M, ncols], for the Q4_K rows W of the
    output columns to check and fp16 activations X [M, K]."""
    X = np.asarray(X)
    if X.dtype != np.float16:
        raise TypeError("X must be float16")
    M, K = X.shape
    if K % QK:
        raise ValueError("K must be a multiple of 256")
    W = _c(W, np.uint8).reshape(-1, K // QK * BLOCK_BYTES)
    ncols = W.shape[0]
    xb = _c(X.view(np.uint16), np.uint16)
    y = np.empty((M, ncols), dtype=np.float64)
    S = np.empty((M, ncols), dtype=np.float64)
    rc = _load().oracle_gemm(W.ctypes.data, xb.ctypes.data, M, ncols, K, y.ctypes.data,
                             S.ctypes.data)
    if rc != 0:
        raise RuntimeError(f"oracle_gemm failed ({rc})")
    return y, S


Q6K_BLOCK_BYTES = 210


def q6k_dequant_rows(W: np.ndarray, K: int) -> np.ndarray:
    """Exact float64 weights [nrows, K] of Q6_K rows W (uint8 [nrows, K/256*210])."""
    W = _c(W, np.uint8)
    nrows = W.size // (K // QK * Q6K_BLOCK_BYTES)
    out = np.empty((nrows, K), dtype=np.float64)
    _load().oracle_q6k_dequant_rows(W.ctypes.data, nrows, K, out.ctypes.data)
    return out


def q6k_gemm(W: np.ndarray, X: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Reference (y, S), both float64 [M, ncols], for the Q6_K rows W of the
    output columns to check and fp16 activations X [M, K]."""
    X = np.asarray(X)
    if X.dtype != np.float16:
        raise TypeError("X must be float16")
    M, K = X.shape
    if K % QK:
        raise ValueError("K must be a multiple of 256")
    W = _c(W, np.uint8).reshape(-1, K // QK * Q6K_BLOCK_BYTES)
    ncols = W.shape[0]
    xb = _c(X.view(np.uint16), np.uint16)
    y = np.empty((M, ncols), dtype=np.float64)
    S = np.empty((M, ncols), dtype=np.float64)
    rc = _load().oracle_q6k_gemm(W.ctypes.data, xb.ctypes.data, M, ncols, K, y.ctypes.data,
                                 S.ctypes.data)
    if rc != 0:
        raise RuntimeError(f"oracle_q6k_gemm failed ({rc})")
    return y, S


def gemm_std(W: np.ndarray, X: np.ndarray, eps: float = 1e-6) -> tuple[np.ndarray, np.ndarray]:
    """Reference (y, S) of one matrix of the layer walk: the Q4_K rows W times
    the row-wise standardized fp16 activations X [M, K] (mean 0, variance 1
    per row, computed exactly in float64, never rounded to binary16)."""
    X = np.asarray(X)
    if X.dtype != np.float16:
        raise TypeError("X must be float16")
    M, K = X.shape
    if K % QK:
        raise ValueError("K must be a multiple of 256")
    W = _c(W, np.uint8).reshape(-1, K // QK * BLOCK_BYTES)
    ncols = W.shape[0]
    xb = _c(X.view(np.uint16), np.uint16)
    y = np.empty((M, ncols), dtype=np.float64)
    S = np.empty((M, ncols), dtype=np.float64)
    rc = _load().oracle_gemm_std(W.ctypes.data, xb.ctypes.data, M, ncols, K, eps,
                                 y.ctypes.data, S.ctypes.data)
    if rc != 0:
        raise RuntimeError(f"oracle_gemm_std failed ({rc})")
    return y, S


def q6k_gemm_std(W: np.ndarray, X: np.ndarray, eps: float = 1e-6) -> tuple[np.ndarray, np.ndarray]:
    """As gemm_std for Q6_K rows W (uint8 [ncols, K/256*210]): the reference of
    a Q6_K matrix (v or down of a Q4_K_M layer) in the layer walk."""
    X = np.asarray(X)
    if X.dtype != np.float16:
        raise TypeError("X must be float16")
    M, K = X.shape
    if K % QK:
        raise ValueError("K must be a multiple of 256")
    W = _c(W, np.uint8).reshape(-1, K // QK * Q6K_BLOCK_BYTES)
    ncols = W.shape[0]
    xb = _c(X.view(np.uint16), np.uint16)
    y = np.empty((M, ncols), dtype=np.float64)
    S = np.empty((M, ncols), dtype=np.float64)
    rc = _load().oracle_q6k_gemm_std(W.ctypes.data, xb.ctypes.data, M, ncols, K, eps,
                                     y.ctypes.data, S.ctypes.data)
    if rc != 0:
        raise RuntimeError(f"oracle_q6k_gemm_std failed ({rc})")
    return y, S


def rms_inv(h: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    """1 / sqrt(mean(h^2) + eps) per row of h [M, N], float64 [M]."""
    h = _c(h, np.float64)
    M, N = h.shape
    out = np.empty(M, dtype=np.float64)
    _load().oracle_rms_inv(h.ctypes.data, M, N, eps, out.ctypes.data)
    return out


def gemm_rms(W: np.ndarray, X: np.ndarray, r: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Reference (y, S) of a normed matrix of the residual walk: the Q4_K rows
    W times the binary16 input X [M, K] scaled per row by r [M]."""
    X = np.asarray(X)
    if X.dtype != np.float16:
        raise TypeError("X must be float16")
    M, K = X.shape
    if K % QK:
        raise ValueError("K must be a multiple of 256")
    W = _c(W, np.uint8).reshape(-1, K // QK * BLOCK_BYTES)
    ncols = W.shape[0]
    xb = _c(X.view(np.uint16), np.uint16)
    r = _c(r, np.float64)
    if r.shape != (M,):
        raise ValueError("r must have one value per row")
    y = np.empty((M, ncols), dtype=np.float64)
    S = np.empty((M, ncols), dtype=np.float64)
    rc = _load().oracle_gemm_rms(W.ctypes.data, xb.ctypes.data, M, ncols, K, r.ctypes.data,
                                 y.ctypes.data, S.ctypes.data)
    if rc != 0:
        raise RuntimeError(f"oracle_gemm_rms failed ({rc})")
    return y, S


def silu(v: np.ndarray) -> np.ndarray:
    """v / (1 + exp(-v)) in float64."""
    v = _c(v, np.float64)
    out = np.empty_like(v)
    _load().oracle_silu(v.ctypes.data, v.size, out.ctypes.data)
    return out


def q8_page(ph) -> tuple[np.ndarray, np.ndarray]:
    """K, V (float64 [16, 128] each) of one 4352-byte page-head of the pool."""
    b = _c(np.frombuffer(bytes(ph), dtype=np.uint8), np.uint8)
    if b.size != 4352:
        raise ValueError("a page-head is 4352 bytes")
    k = np.empty((16, 128), dtype=np.float64)
    v = np.empty((16, 128), dtype=np.float64)
    _load().oracle_q8_page(b.ctypes.data, k.ctypes.data, v.ctypes.data)
    return k, v


def attn_decode(Q, pool, block_table, row_agent, row_len, n_kv: int):
    """Reference (O, S), float64 [M, n_heads, 128], of decode attention over the
    paged q8_0 pool for binary16 queries Q [M, n_heads, 128]; S[d] is
    sum_i p_i |v_i[d]| + 2^-80 * (largest V scale of the attended tokens)."""
    Q = np.asarray(Q)
    if Q.dtype != np.float16 or Q.ndim != 3 or Q.shape[2] != 128:
        raise TypeError("Q must be float16 [M, n_heads, 128]")
    M, H, _ = Q.shape
    qb = _c(Q.view(np.uint16), np.uint16)
    pool = _c(pool, np.uint8)
    bt = _c(block_table, np.int32)
    ra = _c(row_agent, np.int32)
    rl = _c(row_len, np.int32)
    O = np.empty((M, H, 128), dtype=np.float64)
    S = np.empty((M, H, 128), dtype=np.float64)
    rc = _load().oracle_q8_attn(qb.ctypes.data, pool.ctypes.data, bt.ctypes.data, ra.ctypes.data,
                                rl.ctypes.data, M, bt.shape[1], H, n_kv, O.ctypes.data,
                                S.ctypes.data)
    if rc != 0:
        raise RuntimeError(f"oracle_q8_attn failed ({rc})")
    return O, S


def standardize(v: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    """(v - row mean) / sqrt(row variance + eps), float64 [M, N]."""
    v = _c(v, np.float64)
    M, N = v.shape
    out = np.empty_like(v)
    _load().oracle_standardize(v.ctypes.data, M, N, eps, out.ctypes.data)
    return out


def row_moments(v: np.ndarray, eps: float = 1e-6) -> tuple[np.ndarray, np.ndarray]:
    """(mean, 1 / sqrt(variance + eps)) of each row of v [M, N], float64 [M]
    each; a float16 v is taken at its exact binary16 values."""
    v = np.asarray(v)
    if v.dtype == np.float16:
        v = f16_to_f64(v)
    v = _c(v, np.float64)
    M, N = v.shape
    mean = np.empty(M, dtype=np.float64)
    inv = np.empty(M, dtype=np.float64)
    _load().oracle_row_moments(v.ctypes.data, M, N, eps, mean.ctypes.data, inv.ctypes.data)
    return mean, inv


def factored_size(W: np.ndarray, X: np.ndarray, mean=None, r=None) -> np.ndarray:
    """F [M, ncols] float64: the size of the two terms of the factored Q4_K
    weight against binary16 X [M, K],
    r_m * (sum_k (|d sc q| + |dmin m|) |x_mk| + |mean_m * sum_k w_nk|),
    with mean = 0 and r = 1 by default (a plain product)."""
    X = np.asarray(X)
    if X.dtype != np.float16:
        raise TypeError("X must be float16")
    M, K = X.shape
    if K % QK:
        raise ValueError("K must be a multiple of 256")
    W = _c(W, np.uint8).reshape(-1, K // QK * BLOCK_BYTES)
    ncols = W.shape[0]
    xb = _c(X.view(np.uint16), np.uint16)
    mean = _c(np.zeros(M) if mean is None else mean, np.float64)
    r = _c(np.ones(M) if r is None else r, np.float64)
    if mean.shape != (M,) or r.shape != (M,):
        raise ValueError("mean and r must have one value per row")
    F = np.empty((M, ncols), dtype=np.float64)
    rc = _load().oracle_factored_size(W.ctypes.data, xb.ctypes.data, M, ncols, K,
                                      mean.ctypes.data, r.ctypes.data, F.ctypes.data)
    if rc != 0:
        raise RuntimeError(f"oracle_factored_size failed ({rc})")
    return F


def within_bound(y: np.ndarray, y_ref: np.ndarray, S: np.ndarray, tol: float = TOL):
    """Acceptance rule: |y - y_ref| <= tol * S per element, and y exactly 0 where
    S is 0. Returns (ok, worst |err|/S over S>0, number of failing elements)."""
    y = np.asarray(y, dtype=np.float64)
    err = np.abs(y - y_ref)
    zero = S == 0
    bad = (err > tol * S) | (zero & (y != 0)) | ~np.isfinite(y)
    with np.errstate(divide="ignore", invalid="ignore"):
        rel = np.where(zero, 0.0, err / np.where(zero, 1.0, S))
    worst = float(np.max(rel)) if rel.size else 0.0
    return (not bool(bad.any())), worst, int(bad.sum())


def num_threads() -> int:
    """Threads the oracle's parallel loops run on."""
    return int(_load().oracle_num_threads())
