"""The C ABI without a GPU: the library loads, exports every function that
include/mk_q4k.h declares, and rejects bad arguments on the host before any
device access (so these run on CPU-only machines)."""
import ctypes
import os
import re

import pytest

import bit_weight_streaming_amd as mk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mk_q4k.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(mk.LIB_PATH):
        mk.build()
    return mk.lib()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(mk_\w+)\s*\(", src)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for f in ("mk_q4k_gemm", "mk_q4k_gemm_ws", "mk_q4k_gemm_workspace_bytes", "mk_q4k_step",
              "mk_q4k_repack", "mk_q4k_tiles_bytes", "mk_q4k_gemm_tiled",
              "mk_q4k_step_workspace_bytes", "mk_q4k_step_status", "mk_strerror",
              "mk_device_info"):
        assert f in names


def test_every_declared_symbol_is_exported(L):
    for name in declared_functions():
        assert hasattr(L, name), name


def test_strerror_covers_codes(L):
    for code in range(0, -9, -1):
        s = mk.strerror(code)
        assert s and "unknown" not in s
    assert "unknown" in mk.strerror(-1000)


FAKE = 0x7f0000000000   # 16-byte aligned, never dereferenced


def gemm_rc(L, W=FAKE, X=FAKE + (1 << 32), Y=FAKE + (2 << 32), M=12, N=256, K=1024):
    return L.mk_q4k_gemm(W, X, Y, M, N, K, None)


def test_gemm_rejects_bad_shapes(L):
    assert gemm_rc(L, M=0) == mk.MK_EINVAL
    assert gemm_rc(L, M=65) == mk.MK_EINVAL
    assert gemm_rc(L, N=0) == mk.MK_EINVAL
    assert gemm_rc(L, K=0) == mk.MK_EINVAL
    assert gemm_rc(L, K=300) == mk.MK_EINVAL
    assert gemm_rc(L, K=128) == mk.MK_EINVAL


def test_gemm_rejects_null_and_misaligned(L):
    assert gemm_rc(L, W=0) == mk.MK_EINVAL
    assert gemm_rc(L, X=0) == mk.MK_EINVAL
    assert gemm_rc(L, Y=0) == mk.MK_EINVAL
    assert gemm_rc(L, W=FAKE + 8) == mk.MK_EALIGN
    assert gemm_rc(L, X=FAKE + (1 << 32) + 2) == mk.MK_EALIGN
    assert gemm_rc(L, Y=FAKE + (2 << 32) + 4) == mk.MK_EALIGN


def test_gemm_rejects_overlap(L):
    assert gemm_rc(L, Y=FAKE + 16) == mk.MK_EINVAL          # Y inside W
    assert gemm_rc(L, X=FAKE + (2 << 32) + 64) == mk.MK_EINVAL   # X inside Y


def test_gemm_ws_rejects_small_workspace(L):
    need = L.mk_q4k_gemm_workspace_bytes(12, 5120, 17408)
    assert need > 0
    rc = L.mk_q4k_gemm_ws(FAKE, FAKE + (1 << 32), FAKE + (2 << 32), 12, 5120, 17408,
                          FAKE + (3 << 32), need - 1, None)
    assert rc == mk.MK_EWORKSPACE
    rc = L.mk_q4k_gemm_ws(FAKE, FAKE + (1 << 32), FAKE + (2 << 32), 12, 5120, 17408,
                          0, need, None)
    assert rc == mk.MK_EWORKSPACE


def test_workspace_bytes_invalid_is_zero(L):
    assert L.mk_q4k_gemm_workspace_bytes(0, 10, 256) == 0
    assert L.mk_q4k_gemm_workspace_bytes(12, 10, 255) == 0


def test_valid_call_without_gpu_is_nodev(L):
    try:
        import torch
        if torch.cuda.is_available():
            pytest.skip("a GPU is present")
    except ImportError:
        pass
    assert gemm_rc(L) == mk.MK_ENODEV
    buf = ctypes.create_string_buffer(256)
    assert L.mk_device_info(buf, 256) == mk.MK_ENODEV
