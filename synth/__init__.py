"""Seeded synthetic inputs for the Q4_K weight-streaming decode GEMM.

Inputs only: this package generates Q4_K weight blocks and fp16 activation
rows from a counter-based SplitMix64 stream (see ``synth.c`` for the exact
definition). It contains none of the method's arithmetic; the GPU path and the
CPU oracle both consume the bytes it produces and share nothing else.

Workload shapes (the pages' model: a ~27B decoder with hidden size 5120,
64 layers, four agents each stacking one next token and two draft tokens,
so 12 rows per decode step):

* ``TINY``: K=1024, N=256, M=1 (one full oracle check).
* ``GATE_UP``: K=5120, N=17408, M=12.
* ``DOWN``: K=17408, N=5120, M in {1, 4, 8, 12, 16}.
* ``LAYER``: q 5120->6144, k/v 5120->1024, o 6144->5120, gate/up 5120->17408,
  down 17408->5120; 64 layers; M=12.
* ``M64``: the TINY and GATE_UP matrices at M=64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None

BLOCK_BYTES = 144
QK = 256

# Stream tags. A weight matrix of the layer stack is keyed by
# (seed, TAG_WEIGHT, layer, matrix index); activations by (seed, TAG_X, M, K).
TAG_WEIGHT = 1
TAG_X = 2
TAG_COPY = 3   # independent weight copies used to defeat on-chip caches
TAG_NORM = 4   # RMSNorm weights of the residual walk: (seed, TAG_NORM, layer, 0|1)
TAG_H0 = 5     # fp32 residual input of the residual walk: (seed, TAG_H0, M, H)

# Layer stack: (name, K, N) in the order the step walks them.
LAYER_MATRICES = (
    ("q", 5120, 6144),
    ("k", 5120, 1024),
    ("v", 5120, 1024),
    ("o", 6144, 5120),
    ("gate", 5120, 17408),
    ("up", 5120, 17408),
    ("down", 17408, 5120),
)
N_LAYERS = 64
HIDDEN = 5120


def build(force: bool = True) -> str:
    """Compile libsynth.so in place with gcc (OpenMP, -O2, no fast-math)."""
    src = os.path.join(_HERE, "synth.c")
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
        u64 = ctypes.c_uint64
        lib.synth_draw.restype = u64
        lib.synth_draw.argtypes = [u64, u64]
        lib.synth_key.restype = u64
        lib.synth_key.argtypes = [u64, u64, u64, u64]
        lib.synth_q4k_blocks.restype = None
        lib.synth_q4k_blocks.argtypes = [u64, u64, u64, ctypes.c_void_p]
        lib.synth_q4k_rows.restype = None
        lib.synth_q4k_rows.argtypes = [u64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                       ctypes.c_void_p]
        lib.synth_q6k_rows.restype = None
        lib.synth_q6k_rows.argtypes = [u64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                       ctypes.c_void_p]
        lib.synth_q4k_rows_centered.restype = None
        lib.synth_q4k_rows_centered.argtypes = [u64, ctypes.c_int64, ctypes.c_int64,
                                                ctypes.c_int64, ctypes.c_void_p]
        lib.synth_q8_pool.restype = None
        lib.synth_q8_pool.argtypes = [u64, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p]
        lib.synth_f16_normal.restype = None
        lib.synth_f16_normal.argtypes = [u64, u64, u64, ctypes.c_void_p]
        lib.synth_normals.restype = None
        lib.synth_normals.argtypes = [u64, u64, u64, ctypes.c_void_p]
        _lib = lib
    return _lib


def draw(key: int, i: int) -> int:
    return int(_load().synth_draw(key, i))


def key(seed: int, a: int, b: int = 0, c: int = 0) -> int:
    return int(_load().synth_key(seed, a, b, c))


def weight_key(seed: int, layer: int, matrix: int) -> int:
    return key(seed, TAG_WEIGHT, layer, matrix)


def x_key(seed: int, M: int, K: int) -> int:
    return key(seed, TAG_X, M, K)


def q4k_rows(k: int, K: int, n0: int, nrows: int, out: np.ndarray | None = None) -> np.ndarray:
    """Rows [n0, n0+nrows) of the Q4_K matrix of stream k, as uint8 [nrows, K/256*144]."""
    if K % QK:
        raise ValueError("K must be a multiple of 256")
    row_bytes = K // QK * BLOCK_BYTES
    if out is None:
        out = np.empty((nrows, row_bytes), dtype=np.uint8)
    if out.dtype != np.uint8 or not out.flags.c_contiguous or out.size != nrows * row_bytes:
        raise ValueError("out must be a C-contiguous uint8 array of nrows*row_bytes bytes")
    _load().synth_q4k_rows(k, K, n0, nrows, out.ctypes.data)
    return out.reshape(nrows, row_bytes)


def q4k_matrix(k: int, N: int, K: int) -> np.ndarray:
    return q4k_rows(k, K, 0, N)


Q6K_BLOCK_BYTES = 210


def q6k_rows(k: int, K: int, n0: int, nrows: int) -> np.ndarray:
    """Rows [n0, n0+nrows) of the Q6_K matrix of stream k, uint8 [nrows, K/256*210]."""
    if K % QK:
        raise ValueError("K must be a multiple of 256")
    out = np.empty((nrows, K // QK * Q6K_BLOCK_BYTES), dtype=np.uint8)
    _load().synth_q6k_rows(k, K, n0, nrows, out.ctypes.data)
    return out


def q6k_matrix(k: int, N: int, K: int) -> np.ndarray:
    return q6k_rows(k, K, 0, N)


def q4k_rows_centered(k: int, K: int, n0: int, nrows: int) -> np.ndarray:
    """Rows [n0, n0+nrows) of the centred Q4_K matrix of stream k (scales 1..4,
    mins 15*scale, dmin ~ d/2: weights of about zero mean), uint8 [nrows, K/256*144]."""
    if K % QK:
        raise ValueError("K must be a multiple of 256")
    out = np.empty((nrows, K // QK * BLOCK_BYTES), dtype=np.uint8)
    _load().synth_q4k_rows_centered(k, K, n0, nrows, out.ctypes.data)
    return out


def q4k_fill_ptr_centered(k: int, K: int, n0: int, nrows: int, ptr: int) -> None:
    _load().synth_q4k_rows_centered(k, K, n0, nrows, ptr)


def q4k_fill_ptr(k: int, K: int, n0: int, nrows: int, ptr: int) -> None:
    """Write rows [n0, n0+nrows) to host memory at ptr (e.g. a pinned buffer)."""
    _load().synth_q4k_rows(k, K, n0, nrows, ptr)


def f16_normal(k: int, n: int, i0: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.uint16)
    _load().synth_f16_normal(k, i0, n, out.ctypes.data)
    return out.view(np.float16)


def normals(k: int, n: int, i0: int = 0) -> np.ndarray:
    """The float64 normals behind f16_normal (before binary16 rounding)."""
    out = np.empty(n, dtype=np.float64)
    _load().synth_normals(k, i0, n, out.ctypes.data)
    return out


def f32_normal(k: int, n: int, i0: int = 0) -> np.ndarray:
    """float32 of the normals of stream k (round to nearest)."""
    return normals(k, n, i0).astype(np.float32)


# ---- paged q8_0 KV pool for decode attention ----------------------------------
KV_PAGE_TOKENS = 16
KV_HEAD_DIM = 128
KV_PAGE_HEAD_BYTES = 4352
TAG_KV = 6     # (seed, TAG_KV, n_pages, n_kv)


def q8_pool(seed: int, n_pages: int, n_kv: int) -> np.ndarray:
    """uint8 [n_pages, n_kv, 4352]: per page-head the int8 K and V quants of 16
    tokens x 128 dims in four 1 KiB slabs, then binary16 scales per token and
    32-dim block in 64-byte groups of four tokens (offsets in synth.c)."""
    out = np.empty((n_pages, n_kv, KV_PAGE_HEAD_BYTES), dtype=np.uint8)
    _load().synth_q8_pool(key(seed, TAG_KV, n_pages, n_kv), n_pages, n_kv, out.ctypes.data)
    return out


def attn_layout(seed: int, lengths, rows_per_agent: int, n_pages: int):
    """Block tables and rows of a decode step over a shared pool: agent a owns
    ceil(lengths[a] / 16) pages drawn without replacement from a seeded
    permutation of the pool; its rows r = rows_per_agent*a + j attend to the
    first lengths[a] - rows_per_agent + 1 + j tokens (the new tokens are the
    agent's last ones, each row seeing itself and the rows before it).
    Returns (block_table int32 [A, max_pages], row_agent int32 [M],
    row_len int32 [M])."""
    lengths = [int(v) for v in lengths]
    pages = [(n + KV_PAGE_TOKENS - 1) // KV_PAGE_TOKENS for n in lengths]
    if sum(pages) > n_pages:
        raise ValueError("pool too small")
    perm = np.argsort(normals(key(seed, TAG_KV, 1, n_pages), n_pages), kind="stable")
    A = len(lengths)
    table = np.full((A, max(pages)), -1, dtype=np.int32)
    o = 0
    for a in range(A):
        table[a, :pages[a]] = perm[o:o + pages[a]]
        o += pages[a]
    row_agent = np.repeat(np.arange(A, dtype=np.int32), rows_per_agent)
    row_len = np.array([lengths[a] - rows_per_agent + 1 + j for a in range(A)
                        for j in range(rows_per_agent)], dtype=np.int32)
    return table, row_agent, row_len


def activations(seed: int, M: int, K: int) -> np.ndarray:
    """fp16 [M, K] rows of N(0,1) values (row-major, row m = elements m*K..)."""
    return f16_normal(x_key(seed, M, K), M * K).reshape(M, K)
