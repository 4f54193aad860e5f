"""GPU parity of the Q6_K products (mk_q6k_repack + mk_q6k_gemm_tiled, and
mk_q6k_step_repack + mk_q6k_gemm_step) against the fp64 oracle,
|y - y_ref| <= 1e-4 * S per output, S = sum_k |w x|: every output at sizes
spanning several tiles with ragged edges, sampled columns at the full layer
shapes, extreme blocks, and batch invariance (a row's result does not depend
on the other rows in the call)."""
import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)

import bit_weight_streaming_amd as mk  # noqa: E402

DEV = "cuda:0"


def run(W, X, N):
    Wd = torch.from_numpy(np.ascontiguousarray(W)).to(DEV)
    Xd = torch.from_numpy(np.ascontiguousarray(X)).to(DEV)
    T = mk.q6k_repack(Wd, N, X.shape[1])
    Y = mk.q6k_gemm_tiled(T, Xd, N)
    torch.cuda.synchronize()
    return Y.cpu().numpy()


def run_step(W, X, N):
    """The persistent product on the walk-record form."""
    Wd = torch.from_numpy(np.ascontiguousarray(W)).to(DEV)
    Xd = torch.from_numpy(np.ascontiguousarray(X)).to(DEV)
    R = mk.q6k_step_repack(Wd, N, X.shape[1])
    Y = mk.q6k_gemm_step(R, Xd, N)
    torch.cuda.synchronize()
    return Y.cpu().numpy()


def inputs(N, K, M, tag):
    W = synth.q6k_matrix(synth.key(70 + tag, 14, N, K), N, K)
    X = synth.f16_normal(synth.key(70 + tag, 15, M, K), M * K).reshape(M, K)
    return W, X


@pytest.mark.parametrize("M,N,K", [(1, 16, 256), (12, 37, 1024), (16, 100, 2304), (17, 48, 512),
                                   (32, 21, 1280), (5, 333, 4096), (33, 40, 768), (48, 37, 1024),
                                   (64, 100, 2304)])
def test_q6k_all_outputs(M, N, K):
    W, X = inputs(N, K, M, tag=M)
    Y = run(W, X, N)
    y_ref, S = oracle.q6k_gemm(W, X)
    ok, worst, nbad = oracle.within_bound(Y.astype(np.float64), y_ref, S)
    assert ok, f"{nbad} outside the bound, worst {worst:.3e}"
    print(f"M={M} N={N} K={K}: worst |err|/S = {worst:.3e}")


@pytest.mark.parametrize("N,K", [(5120, 17408), (17408, 5120)])
def test_q6k_full_shapes_sampled(N, K):
    """The down and gate/up shapes at M = 12, 512 sampled columns (and the
    first and last) against the oracle."""
    W, X = inputs(N, K, 12, tag=3)
    Y = run(W, X, N)
    cols = np.unique(np.concatenate([np.random.default_rng(9).choice(N, 512, replace=False), [0, N - 1]]))
    y_ref, S = oracle.q6k_gemm(W[cols], X)
    ok, worst, nbad = oracle.within_bound(Y[:, cols].astype(np.float64), y_ref, S)
    assert ok, f"{nbad} outside the bound, worst {worst:.3e}"


def test_q6k_extreme_blocks():
    """Largest binary16 d with scales -128 and 127 and quants 0 and 63, and a
    subnormal d: still within the bound (no overflow in the fp32 sums)."""
    N, K, M = 20, 512, 12
    W, X = inputs(N, K, M, tag=9)
    blocks = W.reshape(N, K // 256, 210)
    blocks[0, :, 208:210] = np.array([6.0e4], dtype=np.float16).view(np.uint8).reshape(1, 2)
    blocks[0, :, 192:208] = np.array([-128, 127] * 8, dtype=np.int8).view(np.uint8)
    blocks[0, :, 0:192] = 0xFF
    blocks[1, :, 208:210] = np.array([2.0 ** -24], dtype=np.float16).view(np.uint8).reshape(1, 2)
    X = (X.astype(np.float32) * np.float32(1e-3)).astype(np.float16)
    Y = run(W, X, N)
    y_ref, S = oracle.q6k_gemm(W, X)
    assert np.all(np.isfinite(Y))
    ok, worst, nbad = oracle.within_bound(Y.astype(np.float64), y_ref, S)
    assert ok, f"{nbad} outside the bound, worst {worst:.3e}"


def test_q6k_rows_bit_identical_alone_or_stacked():
    N, K = 64, 2048
    W, X = inputs(N, K, 12, tag=11)
    Y = run(W, X, N)
    for r in (0, 5, 11):
        one = run(W, X[r:r + 1], N)
        assert np.array_equal(one.view(np.uint32), Y[r:r + 1].view(np.uint32)), r


def test_q6k_rows_past_32_bit_identical():
    """64 rows run as two launches of 32 over the same weights: rows 32.. are,
    bit for bit, what they give alone, and the first 32 what they give as a
    32-row call."""
    N, K = 5120, 2048
    W, X = inputs(N, K, 64, tag=12)
    Y = run(W, X, N)
    first = run(W, X[:32], N)
    rest = run(W, X[32:], N)
    assert np.array_equal(first.view(np.uint32), Y[:32].view(np.uint32))
    assert np.array_equal(rest.view(np.uint32), Y[32:].view(np.uint32))


def test_q6k_rejects_bad_arguments():
    Wd = torch.zeros(32 * 210, dtype=torch.uint8, device=DEV)
    T = mk.q6k_repack(Wd, 32, 256)
    with pytest.raises(mk.MkError) as e:
        mk.q6k_gemm_tiled(T, torch.zeros((65, 256), dtype=torch.float16, device=DEV), 32)
    assert e.value.code == mk.MK_EINVAL


def test_q6k_paired_tiles_odd_count():
    """Enough tiles for two per workgroup (>= 1023), an odd count whose last
    pair lacks its second tile, and a ragged last tile of 2 rows: every
    output against the oracle."""
    N, K, M = 16386, 256, 3
    W, X = inputs(N, K, M, tag=13)
    Y = run(W, X, N)
    y_ref, S = oracle.q6k_gemm(W, X)
    ok, worst, nbad = oracle.within_bound(Y.astype(np.float64), y_ref, S)
    assert ok, f"{nbad} outside the bound, worst {worst:.3e}"


# ---- the persistent product on walk records (mk_q6k_gemm_step)

@pytest.mark.parametrize("M,N,K", [(1, 16, 256), (12, 37, 1024), (16, 100, 2304), (17, 48, 512),
                                   (32, 21, 1280), (5, 333, 4096), (33, 40, 768), (48, 37, 1024),
                                   (64, 100, 2304), (3, 16386, 256)])
def test_q6k_step_records_all_outputs(M, N, K):
    W, X = inputs(N, K, M, tag=M + 40)
    Y = run_step(W, X, N)
    y_ref, S = oracle.q6k_gemm(W, X)
    ok, worst, nbad = oracle.within_bound(Y.astype(np.float64), y_ref, S)
    assert ok, f"{nbad} outside the bound, worst {worst:.3e}"
    print(f"M={M} N={N} K={K}: worst |err|/S = {worst:.3e}")


@pytest.mark.parametrize("M,N,K", [(12, 5120, 17408), (12, 17408, 5120), (64, 5120, 17408)])
def test_q6k_step_records_full_shapes_sampled(M, N, K):
    """The down and gate/up shapes (M = 12, and 64 rows on the down shape), 512
    sampled columns and the first and last against the oracle."""
    W, X = inputs(N, K, M, tag=5)
    Y = run_step(W, X, N)
    cols = np.unique(np.concatenate([np.random.default_rng(19).choice(N, 512, replace=False), [0, N - 1]]))
    y_ref, S = oracle.q6k_gemm(W[cols], X)
    ok, worst, nbad = oracle.within_bound(Y[:, cols].astype(np.float64), y_ref, S)
    assert ok, f"{nbad} outside the bound, worst {worst:.3e}"


def test_q6k_step_records_extreme_blocks():
    """Largest binary16 d with scales -128 and 127 and quants 0 and 63, and a
    subnormal d, as for the tiled product."""
    N, K, M = 20, 512, 12
    W, X = inputs(N, K, M, tag=9)
    blocks = W.reshape(N, K // 256, 210)
    blocks[0, :, 208:210] = np.array([6.0e4], dtype=np.float16).view(np.uint8).reshape(1, 2)
    blocks[0, :, 192:208] = np.array([-128, 127] * 8, dtype=np.int8).view(np.uint8)
    blocks[0, :, 0:192] = 0xFF
    blocks[1, :, 208:210] = np.array([2.0 ** -24], dtype=np.float16).view(np.uint8).reshape(1, 2)
    X = (X.astype(np.float32) * np.float32(1e-3)).astype(np.float16)
    Y = run_step(W, X, N)
    y_ref, S = oracle.q6k_gemm(W, X)
    assert np.all(np.isfinite(Y))
    ok, worst, nbad = oracle.within_bound(Y.astype(np.float64), y_ref, S)
    assert ok, f"{nbad} outside the bound, worst {worst:.3e}"


def test_q6k_step_records_rows_bit_identical_alone_or_stacked():
    """A row's bits do not depend on the rows beside it: 12 decode rows stacked
    with a 32-row chunk (44 rows, three MFMA row tiles) against each part alone
    (one and two row tiles), on a K split into several slices."""
    N, K = 320, 17408
    W, X = inputs(N, K, 44, tag=21)
    Y = run_step(W, X, N)
    dec = run_step(W, X[:12], N)
    chunk = run_step(W, X[12:], N)
    assert np.array_equal(dec.view(np.uint32), Y[:12].view(np.uint32))
    assert np.array_equal(chunk.view(np.uint32), Y[12:].view(np.uint32))
    one = run_step(W, X[7:8], N)
    assert np.array_equal(one.view(np.uint32), Y[7:8].view(np.uint32))


def test_q6k_step_records_deterministic():
    N, K, M = 5120, 2048, 12
    W, X = inputs(N, K, M, tag=23)
    a = run_step(W, X, N)
    b = run_step(W, X, N)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_q6k_step_records_reject_bad_arguments():
    Wd = torch.zeros(32 * 210, dtype=torch.uint8, device=DEV)
    R = mk.q6k_step_repack(Wd, 32, 256)
    with pytest.raises(mk.MkError) as e:
        mk.q6k_gemm_step(R, torch.zeros((65, 256), dtype=torch.float16, device=DEV), 32)
    assert e.value.code == mk.MK_EINVAL
    X = torch.zeros((4, 256), dtype=torch.float16, device=DEV)
    assert mk.lib().mk_q6k_gemm_step(mk._ptr(R), mk._ptr(X), mk._ptr(R), 4, 32, 256, None) == mk.MK_EINVAL
