"""bit_weight_streaming_amd - Q4_K weight-streaming decode GEMM for AMD MI355X.

A thin ctypes binding of ``libmkq4k.so`` (C ABI in ``include/mk_q4k.h``).
PyTorch only allocates device memory and supplies the current HIP stream;
every step of the computation runs in the library's gfx950 kernels. There is
no CPU or PyTorch fallback: if the library is missing or the device is not a
gfx950 GPU, calls raise.

    Y = gemm(W, X)            # W uint8 [N, K/256*144] (Q4_K rows), X fp16 [M, K]
    Wt = repack(W, N, K)      # load-time tile-record form for the step
    step(layers, io, x0, x_out, workspace, M)   # the persistent multi-layer walk
"""
from __future__ import annotations

import ctypes
import os
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))
_ROOT = os.path.dirname(_HERE)
LIB_PATH = os.path.join(_HERE, "libmkq4k.so")
# the same library built with the walk's timeline stamps (a measurement aid,
# bench.py --timeline); the product path never loads it
TIMELINE_LIB_PATH = os.path.join(_HERE, "libmkq4k_timeline.so")
_SOURCES = ["q4k_gemm.hip", "q4k_step.hip", "q4k_repack.hip", "q6k_gemm.hip", "q8_attn.hip",
            "hbm_probe.hip", "mk_api.hip"]
HIPCC_FLAGS = [
    "-O3", "--offload-arch=gfx950", "-fPIC", "-shared", "-std=c++17",
    # packed fp32 instructions stay off (see the build notes)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]

QK = 256
BLOCK_BYTES = 144
MAX_M = 64

MK_OK = 0
MK_EINVAL = -1
MK_EALIGN = -2
MK_EWORKSPACE = -3
MK_EOCCUPANCY = -4
MK_EHIP = -5
MK_ENODEV = -6
MK_ETIMEOUT = -7
MK_ERANGE = -8

_lib = None


class MkError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"mk error {code}: {msg}")
        self.code = code


def sources() -> list[str]:
    return [os.path.join(_HERE, "csrc", s) for s in _SOURCES
            if os.path.exists(os.path.join(_HERE, "csrc", s))]


def build() -> str:
    """Compile libmkq4k.so in place for gfx950 with hipcc (runs without a GPU),
    and libmkq4k_timeline.so, the same sources with the walk's timeline
    stamps (MK_STEP_TIMELINE=1) for bench.py --timeline."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    procs = []
    for path, extra in ((LIB_PATH, []), (TIMELINE_LIB_PATH, ["-DMK_STEP_TIMELINE=1"])):
        cmd = [hipcc, *HIPCC_FLAGS, *extra, "-I", os.path.join(_ROOT, "include"), *sources(), "-o",
               path + ".tmp"]
        procs.append((subprocess.Popen(cmd), path))
    for proc, path in procs:
        if proc.wait() != 0:
            raise subprocess.CalledProcessError(proc.returncode, "hipcc")
    for _, path in procs:
        os.replace(path + ".tmp", path)
    return LIB_PATH


MK_QTYPE_Q4_K = 12
MK_QTYPE_Q6_K = 14


class _Mat(ctypes.Structure):
    _fields_ = [("w", ctypes.c_void_p), ("N", ctypes.c_int), ("K", ctypes.c_int),
                ("type", ctypes.c_int)]


class _Layer(ctypes.Structure):
    _fields_ = [(n, _Mat) for n in ("q", "k", "v", "o", "gate", "up", "down")]


class _LayerIO(ctypes.Structure):
    _fields_ = [("y", ctypes.c_void_p * 7), ("x", ctypes.c_void_p * 4)]


class _LayerResIO(ctypes.Structure):
    _fields_ = [("y", ctypes.c_void_p * 7), ("x", ctypes.c_void_p * 4),
                ("h_mid", ctypes.c_void_p), ("h_out", ctypes.c_void_p)]


class _LayerNorm(ctypes.Structure):
    _fields_ = [("attn", ctypes.c_void_p), ("ffn", ctypes.c_void_p)]


MATRIX_NAMES = ("q", "k", "v", "o", "gate", "up", "down")


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise MkError(MK_ENODEV, f"{LIB_PATH} is missing: run build() first")
        L = ctypes.CDLL(LIB_PATH)
        vp, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        L.mk_strerror.restype = ctypes.c_char_p
        L.mk_strerror.argtypes = [i]
        L.mk_device_info.restype = i
        L.mk_device_info.argtypes = [ctypes.c_char_p, sz]
        L.mk_q4k_gemm.restype = i
        L.mk_q4k_gemm.argtypes = [vp, vp, vp, i, i, i, vp]
        L.mk_q4k_gemm_workspace_bytes.restype = sz
        L.mk_q4k_gemm_workspace_bytes.argtypes = [i, i, i]
        if hasattr(L, "mk_q4k_step_timeline_offset"):
            L.mk_q4k_step_timeline_offset.restype = ctypes.c_longlong
            L.mk_q4k_step_timeline_offset.argtypes = [ctypes.POINTER(_Layer), i, i]
        if hasattr(L, "mk_hbm_read_probe"):
            L.mk_hbm_read_probe.restype = i
            L.mk_hbm_read_probe.argtypes = [vp, sz, vp, i, vp]
        if hasattr(L, "mk_q4k_gemm_noalloc"):
            L.mk_q4k_gemm_noalloc.restype = i
            L.mk_q4k_gemm_noalloc.argtypes = [vp, vp, vp, i, i, i, vp]
        L.mk_q4k_gemm_ws.restype = i
        L.mk_q4k_gemm_ws.argtypes = [vp, vp, vp, i, i, i, vp, sz, vp]
        L.mk_q4k_tiles_bytes.restype = sz
        L.mk_q4k_tiles_bytes.argtypes = [i, i]
        L.mk_q4k_repack.restype = i
        L.mk_q4k_repack.argtypes = [vp, vp, i, i, vp]
        L.mk_q4k_gemm_tiled.restype = i
        L.mk_q4k_gemm_tiled.argtypes = [vp, vp, vp, i, i, i, vp]
        L.mk_q6k_tiles_bytes.restype = sz
        L.mk_q6k_tiles_bytes.argtypes = [i, i]
        L.mk_q6k_repack.restype = i
        L.mk_q6k_repack.argtypes = [vp, vp, i, i, vp]
        L.mk_q6k_step_bytes.restype = sz
        L.mk_q6k_step_bytes.argtypes = [i, i]
        L.mk_q6k_step_repack.restype = i
        L.mk_q6k_step_repack.argtypes = [vp, vp, i, i, vp]
        L.mk_q6k_gemm_tiled.restype = i
        L.mk_q6k_gemm_tiled.argtypes = [vp, vp, vp, i, i, i, vp]
        L.mk_q6k_gemm_step.restype = i
        L.mk_q6k_gemm_step.argtypes = [vp, vp, vp, i, i, i, vp]
        if hasattr(L, "mk_q4k_step"):
            L.mk_q4k_step_workspace_bytes.restype = sz
            L.mk_q4k_step_workspace_bytes.argtypes = [ctypes.POINTER(_Layer), i, i]
            L.mk_q4k_step.restype = i
            L.mk_q4k_step.argtypes = [ctypes.POINTER(_Layer), ctypes.POINTER(_LayerIO), i, i,
                                      vp, vp, vp, sz, vp]
            L.mk_q4k_step_status.restype = i
            L.mk_q4k_step_status.argtypes = [vp, ctypes.POINTER(i)]
            L.mk_q4k_step_set_walk_form.restype = i
            L.mk_q4k_step_set_walk_form.argtypes = [i]
        if hasattr(L, "mk_q8_attn_decode"):
            L.mk_q8_attn_workspace_bytes.restype = sz
            L.mk_q8_attn_workspace_bytes.argtypes = [i, i, i]
            L.mk_q8_attn_decode.restype = i
            L.mk_q8_attn_decode.argtypes = [vp, vp, i, vp, vp, i, i, i, i, i, vp, vp, sz, vp]
        if hasattr(L, "mk_q4k_step_res"):
            L.mk_q4k_step_res.restype = i
            L.mk_q4k_step_res.argtypes = [ctypes.POINTER(_Layer), ctypes.POINTER(_LayerNorm),
                                          ctypes.POINTER(_LayerResIO), i, i, vp, vp, sz, vp]
        _lib = L
    return _lib


def strerror(code: int) -> str:
    return lib().mk_strerror(code).decode()


def _check(rc: int) -> None:
    if rc != MK_OK:
        raise MkError(rc, strerror(rc))


def device_info() -> str:
    buf = ctypes.create_string_buffer(1024)
    _check(lib().mk_device_info(buf, len(buf)))
    return buf.value.decode()


def _stream(stream=None) -> int:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


def _ptr(t) -> int:
    return int(t.data_ptr()) if t is not None else 0


def gemm(W, X, out=None, stream=None, workspace=None):
    """Y = X * W^T. W: uint8 [N, K/256*144] (or flat), X: float16 [M, K], both on
    the GPU; returns float32 [M, N] (written into `out` if given). A
    `workspace` (uint8 device tensor of gemm_workspace_bytes) needs no
    initial contents; each call overwrites what it uses."""
    import torch
    if X.dim() != 2 or X.dtype != torch.float16:
        raise MkError(MK_EINVAL, "X must be a 2-D float16 tensor")
    M, K = X.shape
    if K % QK:
        raise MkError(MK_EINVAL, "K must be a multiple of 256")
    if W.dtype != torch.uint8 or W.numel() % (K // QK * BLOCK_BYTES):
        raise MkError(MK_EINVAL, "W must be uint8 Q4_K rows of K/256*144 bytes")
    if not (X.is_contiguous() and W.is_contiguous()):
        raise MkError(MK_EINVAL, "W and X must be contiguous")
    N = W.numel() // (K // QK * BLOCK_BYTES)
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=X.device)
    elif out.shape != (M, N) or out.dtype != torch.float32 or not out.is_contiguous():
        raise MkError(MK_EINVAL, "out must be a contiguous float32 [M, N] tensor")
    if workspace is None:
        rc = lib().mk_q4k_gemm(_ptr(W), _ptr(X), _ptr(out), M, N, K, _stream(stream))
    else:
        rc = lib().mk_q4k_gemm_ws(_ptr(W), _ptr(X), _ptr(out), M, N, K, _ptr(workspace),
                                  workspace.numel() * workspace.element_size(), _stream(stream))
    _check(rc)
    return out


def hbm_read_probe(buf, out, grid: int, stream=None):
    """Read every byte of the device tensor `buf` once (16-byte nontemporal
    loads, `grid` workgroups of 512 threads, one contiguous share each) and
    write one XOR word per workgroup into `out` (uint32/int32, >= grid
    entries): the read bandwidth the chip reaches, for the measured ceiling."""
    if out.numel() < grid or out.element_size() != 4:
        raise MkError(MK_EINVAL, "out needs one 32-bit word per workgroup")
    _check(lib().mk_hbm_read_probe(_ptr(buf), buf.numel() * buf.element_size(), _ptr(out), grid,
                                   _stream(stream)))


def gemm_noalloc(W, X, out=None, stream=None):
    """Y = X * W^T like gemm(), through mk_q4k_gemm_noalloc: the K-split
    partials go to the library's static per-GPU scratch array (calls that
    overlap on one GPU race); shapes that need more than it holds raise
    MkError(MK_EWORKSPACE)."""
    import torch
    if X.dim() != 2 or X.dtype != torch.float16 or not X.is_contiguous():
        raise MkError(MK_EINVAL, "X must be a contiguous 2-D float16 tensor")
    M, K = X.shape
    if K % QK or W.dtype != torch.uint8 or W.numel() % (K // QK * BLOCK_BYTES) \
            or not W.is_contiguous():
        raise MkError(MK_EINVAL, "W must be contiguous uint8 Q4_K rows of K/256*144 bytes")
    N = W.numel() // (K // QK * BLOCK_BYTES)
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=X.device)
    elif out.shape != (M, N) or out.dtype != torch.float32 or not out.is_contiguous():
        raise MkError(MK_EINVAL, "out must be a contiguous float32 [M, N] tensor")
    _check(lib().mk_q4k_gemm_noalloc(_ptr(W), _ptr(X), _ptr(out), M, N, K, _stream(stream)))
    return out


def gemm_tiled(Wt, X, N: int, out=None, stream=None):
    """Y = X * W^T with W in the tile-record form (repack()); N columns."""
    import torch
    if X.dim() != 2 or X.dtype != torch.float16 or not X.is_contiguous():
        raise MkError(MK_EINVAL, "X must be a contiguous 2-D float16 tensor")
    M, K = X.shape
    nbytes = tiles_bytes(N, K)
    if nbytes == 0 or Wt.dtype != torch.uint8 or Wt.numel() < nbytes or not Wt.is_contiguous():
        raise MkError(MK_EINVAL, "Wt must be the contiguous tile-record form of an N x K matrix")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=X.device)
    elif out.shape != (M, N) or out.dtype != torch.float32 or not out.is_contiguous():
        raise MkError(MK_EINVAL, "out must be a contiguous float32 [M, N] tensor")
    _check(lib().mk_q4k_gemm_tiled(_ptr(Wt), _ptr(X), _ptr(out), M, N, K, _stream(stream)))
    return out


def gemm_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(lib().mk_q4k_gemm_workspace_bytes(M, N, K))


def tiles_bytes(N: int, K: int) -> int:
    """Bytes of the tile-record form of an N x K Q4_K matrix."""
    return int(lib().mk_q4k_tiles_bytes(N, K))


def repack(W, N: int, K: int, out=None, stream=None):
    """Tile-record form (uint8 device tensor) of the Q4_K rows W (device)."""
    import torch
    nbytes = tiles_bytes(N, K)
    if nbytes == 0:
        raise MkError(MK_EINVAL, "invalid shape")
    if W.dtype != torch.uint8 or W.numel() != N * (K // QK) * BLOCK_BYTES or not W.is_contiguous():
        raise MkError(MK_EINVAL, "W must be contiguous uint8 Q4_K rows")
    if out is None:
        out = torch.empty(nbytes, dtype=torch.uint8, device=W.device)
    elif out.numel() * out.element_size() < nbytes or not out.is_contiguous():
        raise MkError(MK_EINVAL, "out too small")
    _check(lib().mk_q4k_repack(_ptr(W), _ptr(out), N, K, _stream(stream)))
    return out


Q6K_BLOCK_BYTES = 210


def q6k_tiles_bytes(N: int, K: int) -> int:
    """Bytes of the tile-record form of an N x K Q6_K matrix."""
    return int(lib().mk_q6k_tiles_bytes(N, K))


def q6k_repack(W, N: int, K: int, out=None, stream=None):
    """Tile-record form (uint8 device tensor) of the Q6_K rows W (device)."""
    import torch
    nbytes = q6k_tiles_bytes(N, K)
    if nbytes == 0:
        raise MkError(MK_EINVAL, "invalid shape")
    if W.dtype != torch.uint8 or W.numel() != N * (K // QK) * Q6K_BLOCK_BYTES or not W.is_contiguous():
        raise MkError(MK_EINVAL, "W must be contiguous uint8 Q6_K rows")
    if out is None:
        out = torch.empty(nbytes, dtype=torch.uint8, device=W.device)
    elif out.numel() * out.element_size() < nbytes or not out.is_contiguous():
        raise MkError(MK_EINVAL, "out too small")
    _check(lib().mk_q6k_repack(_ptr(W), _ptr(out), N, K, _stream(stream)))
    return out


def q6k_step_bytes(N: int, K: int) -> int:
    """Bytes of the walk-record form of an N x K Q6_K matrix (records + column sums)."""
    return int(lib().mk_q6k_step_bytes(N, K))


def q6k_step_repack(W, N: int, K: int, out=None, stream=None):
    """Walk-record form (uint8 device tensor) of the Q6_K rows W (device), for a
    step matrix of type MK_QTYPE_Q6_K."""
    import torch
    nbytes = q6k_step_bytes(N, K)
    if nbytes == 0:
        raise MkError(MK_EINVAL, "invalid shape")
    if W.dtype != torch.uint8 or W.numel() != N * (K // QK) * Q6K_BLOCK_BYTES or not W.is_contiguous():
        raise MkError(MK_EINVAL, "W must be contiguous uint8 Q6_K rows")
    if out is None:
        out = torch.empty(nbytes, dtype=torch.uint8, device=W.device)
    elif out.numel() * out.element_size() < nbytes or not out.is_contiguous():
        raise MkError(MK_EINVAL, "out too small")
    _check(lib().mk_q6k_step_repack(_ptr(W), _ptr(out), N, K, _stream(stream)))
    return out


def q6k_gemm_tiled(Wt, X, N: int, out=None, stream=None):
    """Y = X * W^T with the Q6_K matrix W in tile-record form (q6k_repack()); N columns."""
    import torch
    if X.dim() != 2 or X.dtype != torch.float16 or not X.is_contiguous():
        raise MkError(MK_EINVAL, "X must be a contiguous 2-D float16 tensor")
    M, K = X.shape
    nbytes = q6k_tiles_bytes(N, K)
    if nbytes == 0 or Wt.dtype != torch.uint8 or Wt.numel() < nbytes or not Wt.is_contiguous():
        raise MkError(MK_EINVAL, "Wt must be the contiguous tile-record form of an N x K Q6_K matrix")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=X.device)
    elif out.shape != (M, N) or out.dtype != torch.float32 or not out.is_contiguous():
        raise MkError(MK_EINVAL, "out must be a contiguous float32 [M, N] tensor")
    _check(lib().mk_q6k_gemm_tiled(_ptr(Wt), _ptr(X), _ptr(out), M, N, K, _stream(stream)))
    return out


def q6k_gemm_step(Ws, X, N: int, out=None, stream=None):
    """Y = X * W^T with the Q6_K matrix W in walk-record form (q6k_step_repack());
    N columns; the persistent K-split product."""
    import torch
    if X.dim() != 2 or X.dtype != torch.float16 or not X.is_contiguous():
        raise MkError(MK_EINVAL, "X must be a contiguous 2-D float16 tensor")
    M, K = X.shape
    nbytes = q6k_step_bytes(N, K)
    if nbytes == 0 or Ws.dtype != torch.uint8 or Ws.numel() < nbytes or not Ws.is_contiguous():
        raise MkError(MK_EINVAL, "Ws must be the contiguous walk-record form of an N x K Q6_K matrix")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=X.device)
    elif out.shape != (M, N) or out.dtype != torch.float32 or not out.is_contiguous():
        raise MkError(MK_EINVAL, "out must be a contiguous float32 [M, N] tensor")
    _check(lib().mk_q6k_gemm_step(_ptr(Ws), _ptr(X), _ptr(out), M, N, K, _stream(stream)))
    return out


# ---------------------------------------------------------------- the step

def _layers_struct(layers):
    arr = (_Layer * len(layers))()
    for i, lay in enumerate(layers):
        for name in MATRIX_NAMES:
            # (W, N, K) for a Q4_K matrix, (W, N, K, type) in general
            w, n, k, *t = lay[name]
            qt = t[0] if t else MK_QTYPE_Q4_K
            setattr(arr[i], name, _Mat(_ptr(w) if not isinstance(w, int) else w, n, k, qt))
    return arr


def step_workspace_bytes(layer0, n_layers: int, M: int) -> int:
    arr = _layers_struct([layer0])
    return int(lib().mk_q4k_step_workspace_bytes(arr, n_layers, M))


def step_timeline_offset(layer0, n_layers: int, M: int) -> int:
    """Byte offset of the walk's timeline stamps in its workspace (a library
    loaded from TIMELINE_LIB_PATH), or -1 for the product library."""
    arr = _layers_struct([layer0])
    return int(lib().mk_q4k_step_timeline_offset(arr, n_layers, M))


def step(layers, io, x0, x_out, workspace, M: int, stream=None) -> None:
    """Enqueue the persistent walk. layers: list of dicts name -> (W tensor,
    N, K); io: list of dicts with 'y' (7 float32 tensors, matrix order) and
    'x' (4 float16 tensors, phase inputs A..D)."""
    larr = _layers_struct(layers)
    ioarr = (_LayerIO * len(io))()
    for i, d in enumerate(io):
        for t in range(7):
            ioarr[i].y[t] = _ptr(d["y"][t])
        for p in range(4):
            ioarr[i].x[p] = _ptr(d["x"][p])
    rc = lib().mk_q4k_step(larr, ioarr, len(layers), M, _ptr(x0), _ptr(x_out), _ptr(workspace),
                           workspace.numel() * workspace.element_size(), _stream(stream))
    _check(rc)


def step_res(layers, io, norms, h0, workspace, M: int, stream=None) -> None:
    """Enqueue the residual walk. layers as for step(); io: list of dicts with
    'y' (7 float32 tensors), 'x' (4 float16 tensors) and 'h' (2 float32 [M, H]
    tensors: the residual after o and after down); norms: list of pairs of
    float32 [H] tensors (before q/k/v, before gate/up); h0: float32 [M, H]."""
    larr = _layers_struct(layers)
    ioarr = (_LayerResIO * len(io))()
    narr = (_LayerNorm * len(norms))()
    for i, d in enumerate(io):
        for t in range(7):
            ioarr[i].y[t] = _ptr(d["y"][t])
        for p in range(4):
            ioarr[i].x[p] = _ptr(d["x"][p])
        ioarr[i].h_mid = _ptr(d["h"][0])
        ioarr[i].h_out = _ptr(d["h"][1])
    for i, (a, f) in enumerate(norms):
        narr[i].attn = _ptr(a)
        narr[i].ffn = _ptr(f)
    rc = lib().mk_q4k_step_res(larr, narr, ioarr, len(layers), M, _ptr(h0), _ptr(workspace),
                               workspace.numel() * workspace.element_size(), _stream(stream))
    _check(rc)


def attn_workspace_bytes(n_agents: int, max_pages: int, n_kv: int) -> int:
    return int(lib().mk_q8_attn_workspace_bytes(n_agents, max_pages, n_kv))


def attn_decode(Q, pool, block_table, row_len, rows_per_agent: int, n_kv: int, workspace=None,
                out=None, stream=None):
    """Decode attention over the paged q8_0 pool. Q: float16 [M, n_heads, 128];
    pool: uint8 [n_pages, n_kv, 4352]; block_table: int32 [n_agents, max_pages];
    row_len: int32 [M] (all device tensors). Returns float32 [M, n_heads, 128]."""
    import torch
    M, H, D = Q.shape
    A, P = block_table.shape
    if D != 128 or Q.dtype != torch.float16 or M != A * rows_per_agent:
        raise MkError(MK_EINVAL, "Q must be float16 [n_agents * rows_per_agent, n_heads, 128]")
    if pool.dtype != torch.uint8 or pool.numel() % (n_kv * 4352):
        raise MkError(MK_EINVAL, "pool must be uint8 pages of n_kv * 4352 bytes")
    if block_table.dtype != torch.int32 or row_len.dtype != torch.int32 or row_len.numel() != M:
        raise MkError(MK_EINVAL, "block_table and row_len must be int32")
    for t in (Q, pool, block_table, row_len):
        if not t.is_contiguous():
            raise MkError(MK_EINVAL, "inputs must be contiguous")
    if out is None:
        out = torch.empty((M, H, 128), dtype=torch.float32, device=Q.device)
    if workspace is None:
        workspace = torch.empty(max(attn_workspace_bytes(A, P, n_kv), 16), dtype=torch.uint8,
                                device=Q.device)
    rc = lib().mk_q8_attn_decode(_ptr(Q), _ptr(pool), pool.numel() // (n_kv * 4352),
                                 _ptr(block_table), _ptr(row_len), A, rows_per_agent, P, H, n_kv,
                                 _ptr(out), _ptr(workspace),
                                 workspace.numel() * workspace.element_size(), _stream(stream))
    _check(rc)
    return out


MK_WALK_AUTO = 0
MK_WALK_ITERATOR = 1
MK_WALK_RELOAD_STATS = 2


def step_set_walk_form(form: int) -> None:
    """Testing aid (flags, OR-ed): MK_WALK_ITERATOR makes later walks use the
    record iterator instead of the per-wave record tables; MK_WALK_RELOAD_STATS
    makes every phase reload its input statistics at the end of its compute.
    The results are the same, bit for bit."""
    _check(lib().mk_q4k_step_set_walk_form(int(form)))


def step_status(workspace) -> int:
    st = ctypes.c_int(0)
    _check(lib().mk_q4k_step_status(_ptr(workspace), ctypes.byref(st)))
    return st.value
