"""The C ABI without a GPU: the library loads, exports every function that
the headers in include/ declare, and rejects bad arguments on the host before any
device access (so these run on CPU-only machines)."""
import ctypes
import os
import re

import pytest

import bit_weight_streaming_amd as mk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", f) for f in sorted(os.listdir(os.path.join(ROOT, "include")))
           if f.endswith(".h")]


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(mk.LIB_PATH):
        mk.build()
    return mk.lib()


def declared_functions():
    src = "".join(open(h).read() for h in HEADERS)
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(mk_\w+)\s*\(", src)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for f in ("mk_q4k_gemm", "mk_q4k_gemm_ws", "mk_q4k_gemm_workspace_bytes", "mk_q4k_step",
              "mk_q4k_repack", "mk_q4k_tiles_bytes", "mk_q4k_gemm_tiled",
              "mk_q4k_step_workspace_bytes", "mk_q4k_step_status", "mk_strerror",
              "mk_device_info", "mk_q4k_step_res", "mk_q8_attn_decode",
              "mk_q8_attn_workspace_bytes", "mk_q4k_gemm_noalloc"):
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


def test_attn_rejects_bad_arguments(L):
    ws = FAKE + (3 << 32)
    args = dict(Q=FAKE, pool=FAKE + (1 << 32), n_pages=10, table=FAKE + (2 << 32),
                lens=FAKE + (4 << 32), A=4, R=3, P=8, H=48, KV=8, O=FAKE + (5 << 32))

    def rc(**kw):
        a = dict(args, **kw)
        return L.mk_q8_attn_decode(a["Q"], a["pool"], a["n_pages"], a["table"], a["lens"],
                                   a["A"], a["R"], a["P"], a["H"], a["KV"], a["O"], ws,
                                   1 << 30, None)
    assert rc(H=47) == mk.MK_EINVAL          # heads not a multiple of KV heads
    assert rc(R=6) == mk.MK_EINVAL           # 6 rows x 6 heads per KV head > 32
    assert rc(n_pages=0) == mk.MK_EINVAL
    assert rc(Q=FAKE + 2) == mk.MK_EALIGN
    assert L.mk_q8_attn_decode(FAKE, FAKE + (1 << 32), 10, FAKE + (2 << 32), FAKE + (4 << 32),
                               4, 3, 8, 48, 8, FAKE + (5 << 32), ws, 16, None) == mk.MK_EWORKSPACE
    assert L.mk_q8_attn_workspace_bytes(4, 8, 8) == 4 * 8 * 1 * 32 * 132 * 4


def test_q6k_rejects_bad_arguments(L):
    T, X, Y = FAKE, FAKE + (1 << 32), FAKE + (2 << 32)
    assert L.mk_q6k_tiles_bytes(16, 256) == 3360
    assert L.mk_q6k_tiles_bytes(17, 512) == 2 * 2 * 3360
    assert L.mk_q6k_tiles_bytes(16, 300) == 0 and L.mk_q6k_tiles_bytes(0, 256) == 0
    assert L.mk_q6k_gemm_tiled(T, X, Y, 65, 16, 256, None) == mk.MK_EINVAL    # M > 64
    assert L.mk_q6k_gemm_tiled(T, X, Y, 0, 16, 256, None) == mk.MK_EINVAL
    assert L.mk_q6k_gemm_tiled(T, X, Y, 4, 16, 200, None) == mk.MK_EINVAL    # K % 256
    assert L.mk_q6k_gemm_tiled(None, X, Y, 4, 16, 256, None) == mk.MK_EINVAL
    assert L.mk_q6k_gemm_tiled(T, X + 8, Y, 4, 16, 256, None) == mk.MK_EALIGN
    assert L.mk_q6k_repack(None, T, 16, 256, None) == mk.MK_EINVAL
    assert L.mk_q6k_repack(X, T + 4, 16, 256, None) == mk.MK_EALIGN


# --- the walk's index arithmetic, checked on the host ---------------------------
def _layer(shp):
    lay = mk._Layer()
    for name in mk.MATRIX_NAMES:
        N, K = shp[name]
        m = getattr(lay, name)
        m.w, m.N, m.K = None, N, K
    return lay


def _plan_violations(L, shp, n_layers, M, G):
    L.mk_q4k_step_check_plan.restype = ctypes.c_longlong
    L.mk_q4k_step_check_plan.argtypes = [ctypes.POINTER(mk._Layer), ctypes.c_int, ctypes.c_int,
                                         ctypes.c_int]
    lay = _layer(shp)
    return L.mk_q4k_step_check_plan(ctypes.byref(lay), n_layers, M, G)


@pytest.mark.parametrize("G", [256, 304, 228, 120, 80])
def test_step_plan_accesses_stay_in_bounds(L, G):
    """For every shape the tests and the benchmark walk, at several compute
    unit counts, every weight record, column sum, slice partial, LDS slot,
    staged row, finishing tile and statistics slot the kernel's index
    arithmetic reaches lies inside its buffer, and every tile is covered and
    finished exactly once (a host walk with the kernel's own split functions)."""
    from synth.stack import shapes
    cases = [shapes(), shapes(H=512, Nq=768, Nkv=256, F=1280), shapes(H=768, Nq=512, Nkv=200, F=1024),
             shapes(H=256, Nq=256, Nkv=16, F=512)]
    for shp in cases:
        for M in (1, 5, 12, 16, 33, 64):
            for n_layers in (1, 3, 64):
                v = _plan_violations(L, shp, n_layers, M, G)
                # -1: no plan fits (the launch refuses it); MI355X's 256 CUs fit all
                assert v == 0 or (v == -1 and G != 256), (shp["q"], shp["gate"], M, n_layers, G, v)


def test_step_plan_check_rejects_bad_shapes(L):
    from synth.stack import shapes
    bad = shapes()
    bad["o"] = (5120, 6000)          # o.K != q.N, and not a multiple of 256
    assert _plan_violations(L, bad, 1, 12, 256) == mk.MK_EINVAL
    assert _plan_violations(L, shapes(), 1, 65, 256) == mk.MK_EINVAL
    assert _plan_violations(L, shapes(), 1, 0, 256) == mk.MK_EINVAL
    assert _plan_violations(L, shapes(), 1, 12, 0) == mk.MK_EINVAL


def test_step_workspace_is_one_row_group(L):
    """Rows past 16 run as further walks over row groups of 16, one after
    another in the same workspace: a call of up to 64 rows needs the
    workspace of 16 rows, and 65 rows are refused (size 0)."""
    from synth.stack import shapes
    L.mk_q4k_step_workspace_bytes.restype = ctypes.c_size_t
    L.mk_q4k_step_workspace_bytes.argtypes = [ctypes.POINTER(mk._Layer), ctypes.c_int, ctypes.c_int]
    lay = _layer(shapes())
    w16 = L.mk_q4k_step_workspace_bytes(ctypes.byref(lay), 64, 16)
    assert w16 > 0
    for M in (17, 32, 44, 64):
        assert L.mk_q4k_step_workspace_bytes(ctypes.byref(lay), 64, M) == w16
    assert L.mk_q4k_step_workspace_bytes(ctypes.byref(lay), 64, 65) == 0


def test_step_rejects_q6k_outside_v_and_down(L):
    """Only v and down may be Q6_K (what a Q4_K_M file keeps in Q6_K)."""
    from synth.stack import shapes
    for name in ("q", "k", "o", "gate", "up"):
        lay = _layer(shapes())
        getattr(lay, name).type = mk.MK_QTYPE_Q6_K
        assert L.mk_q4k_step_check_plan(ctypes.byref(lay), 1, 12, 256) == mk.MK_EINVAL, name
    lay = _layer(shapes())
    lay.v.type = mk.MK_QTYPE_Q6_K
    lay.down.type = mk.MK_QTYPE_Q6_K
    assert L.mk_q4k_step_check_plan(ctypes.byref(lay), 1, 12, 256) == 0
    lay.down.type = 3                                     # not a supported type
    assert L.mk_q4k_step_check_plan(ctypes.byref(lay), 1, 12, 256) == mk.MK_EINVAL


def test_q6k_step_bytes(L):
    L.mk_q6k_step_bytes.restype = ctypes.c_size_t
    L.mk_q6k_step_bytes.argtypes = [ctypes.c_int, ctypes.c_int]
    assert L.mk_q6k_step_bytes(16, 256) == 3360 + 16 * 4
    assert L.mk_q6k_step_bytes(17, 512) == 2 * 2 * 3360 + 32 * 4
    assert L.mk_q6k_step_bytes(16, 300) == 0 and L.mk_q6k_step_bytes(0, 256) == 0


def test_walk_form_switch_on_the_host(L):
    """The walk-form switch needs no device: it takes the documented flags,
    alone or together, and refuses other bits (the GPU tests compare the
    forms)."""
    L.mk_q4k_step_set_walk_form.restype = ctypes.c_int
    L.mk_q4k_step_set_walk_form.argtypes = [ctypes.c_int]
    assert L.mk_q4k_step_set_walk_form(4) == mk.MK_EINVAL
    assert L.mk_q4k_step_set_walk_form(-1) == mk.MK_EINVAL
    assert L.mk_q4k_step_set_walk_form(mk.MK_WALK_ITERATOR) == 0
    assert L.mk_q4k_step_set_walk_form(mk.MK_WALK_RELOAD_STATS) == 0
    assert L.mk_q4k_step_set_walk_form(mk.MK_WALK_ITERATOR | mk.MK_WALK_RELOAD_STATS) == 0
    assert L.mk_q4k_step_set_walk_form(mk.MK_WALK_AUTO) == 0
