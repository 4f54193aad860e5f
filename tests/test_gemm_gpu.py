"""GPU parity of mk_q4k_gemm against the fp64 oracle, plus the properties the
kernel must keep (determinism, exact scaling, row permutation), edge cases and
the single-matrix workloads at their full sizes. Every call goes through the
C ABI (libmkq4k.so) via the ctypes binding."""
import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU containers
    pytest.skip("needs a GPU", allow_module_level=True)

import bit_weight_streaming_amd as mk  # noqa: E402

DEV = "cuda:0"


def run_gpu(W_np, X_np):
    W = torch.from_numpy(np.ascontiguousarray(W_np)).to(DEV)
    X = torch.from_numpy(np.ascontiguousarray(X_np)).to(DEV)
    Y = mk.gemm(W, X)
    torch.cuda.synchronize()
    return Y.cpu().numpy()


def check(W_np, X_np, cols=None, Y=None):
    """Parity within |y - y_ref| <= 1e-4 * S on all columns or on `cols`."""
    if Y is None:
        Y = run_gpu(W_np, X_np)
    Wc = W_np if cols is None else W_np[cols]
    y_ref, S = oracle.gemm(Wc, X_np)
    Yc = Y if cols is None else Y[:, cols]
    ok, worst, nbad = oracle.within_bound(Yc, y_ref, S)
    assert ok, f"{nbad} elements outside the bound, worst |err|/S = {worst:.3e}"
    return Y, worst


def inputs(N, K, M, seed=0, tag=0):
    W = synth.q4k_matrix(synth.key(seed, synth.TAG_WEIGHT, tag, N * 100003 + K), N, K)
    X = synth.activations(seed + tag, M, K)
    return W, X


def test_device_is_gfx950():
    info = mk.device_info()
    assert "gfx950" in info


# --- the tiny workload: K=1024, N=256, M=1, seed 0, every column ----------------
def test_tiny_all_columns():
    W = synth.q4k_matrix(synth.weight_key(0, 0, 0), 256, 1024)
    X = synth.activations(0, 1, 1024)
    _, worst = check(W, X)
    print(f"tiny worst |err|/S = {worst:.3e}")


# --- shapes that span several tiles, a ragged tail and every row-tile count -----
@pytest.mark.parametrize("M,N,K", [
    (1, 257, 768), (5, 257, 1024), (12, 100, 2560), (16, 33, 512), (17, 48, 1280),
    (31, 40, 256), (32, 17, 1536), (33, 64, 768), (48, 16, 512), (49, 31, 1024),
    (64, 70, 2048), (12, 1, 256), (3, 15, 4096),
])
def test_parity_shapes(M, N, K):
    W, X = inputs(N, K, M, tag=M)
    check(W, X)


# --- the single-projection workload: K=5120, N=17408, M=12, every column --------
def test_gate_up_m12_full():
    W, X = inputs(17408, 5120, 12, tag=2)
    _, worst = check(W, X)
    print(f"gate/up M=12 worst |err|/S = {worst:.3e}")


# --- the down-projection sweep: K=17408, N=5120, M in {1,4,8,12,16} -------------
@pytest.mark.parametrize("M", [1, 4, 8, 12, 16])
def test_down_sweep_full(M):
    W, X = inputs(5120, 17408, M, tag=3)
    check(W, X)


# --- 64 rows on both single-matrix shapes ---------------------------------------
def test_m64_tiny_full():
    W = synth.q4k_matrix(synth.weight_key(0, 0, 0), 256, 1024)
    X = synth.activations(5, 64, 1024)
    check(W, X)


def test_m64_gate_up_sampled():
    W, X = inputs(17408, 5120, 64, tag=5)
    rng = np.random.default_rng(5)
    cols = np.sort(rng.choice(17408, 3000, replace=False))
    cols = np.unique(np.concatenate([cols, [0, 15, 16, 17407]]))
    check(W, X, cols=cols)


# --- edge cases -----------------------------------------------------------------
def test_all_zero_weights_give_exact_zero():
    W = np.zeros((40, 4 * 144), dtype=np.uint8)
    X = synth.activations(1, 9, 1024)
    Y = run_gpu(W, X)
    assert np.all(Y == 0)


def test_zero_activations_give_exact_zero():
    W, _ = inputs(50, 1024, 3, tag=7)
    X = np.zeros((3, 1024), dtype=np.float16)
    Y = run_gpu(W, X)
    assert np.all(Y == 0)


def _blocks(d_bits, dmin_bits, scale_byte, q_byte, n_rows, kb):
    blk = bytearray(144)
    blk[0:2] = d_bits.to_bytes(2, "little")
    blk[2:4] = dmin_bits.to_bytes(2, "little")
    blk[4:16] = bytes([scale_byte] * 12)
    blk[16:] = bytes([q_byte] * 128)
    return np.frombuffer(bytes(blk) * (n_rows * kb), dtype=np.uint8).reshape(n_rows, kb * 144)


def test_max_scale_blocks():
    W = _blocks(0x3C00, 0x3C00, 0xFF, 0xFF, 20, 2)      # every w = 882
    X = synth.activations(2, 4, 512)
    check(W, X)


def test_subnormal_d_and_dmin():
    # d = 3 * 2^-24, dmin = 2^-24 on every block, random nibbles/scales
    W, X = inputs(64, 1024, 6, tag=9)
    W = W.copy().reshape(-1, 144)
    W[:, 0:2] = np.frombuffer((3).to_bytes(2, "little"), dtype=np.uint8)
    W[:, 2:4] = np.frombuffer((1).to_bytes(2, "little"), dtype=np.uint8)
    W = W.reshape(64, -1)
    Y, _ = check(W, X)
    assert np.count_nonzero(Y) > 0


def test_subnormal_activations():
    W, _ = inputs(48, 768, 5, tag=10)
    rng = np.random.default_rng(3)
    bits = rng.integers(1, 1024, size=(5, 768)).astype(np.uint16)    # subnormal fp16
    bits |= (rng.integers(0, 2, size=(5, 768)).astype(np.uint16) << 15)
    X = bits.view(np.float16)
    Y, _ = check(W, X)
    assert np.count_nonzero(Y) > 0


def test_min_only_blocks():
    W = _blocks(0x3C00, 0x3800, 0x2A, 0x00, 30, 3)      # q = 0: w = -dmin * m
    X = synth.activations(3, 7, 768)
    check(W, X)


def test_large_activation_values():
    W, _ = inputs(32, 512, 4, tag=11)
    X = (synth.activations(4, 4, 512).astype(np.float32) * 1000).astype(np.float16)
    check(W, X)


# --- the min term's sub-block sums and nearly cancelling weights ------------------
def _big_sum_rows(M, K, seed):
    """N(0,1) rows with whole 32-value sub-blocks of large values: 2100 (sum
    67200, past binary16's 65504), -2100, 65504 (the largest finite value, sum
    2096128) and -30000, at different sub-blocks per row."""
    X = synth.activations(seed, M, K).astype(np.float32)
    for m in range(M):
        for i, v in enumerate((2100.0, -2100.0, 65504.0, -30000.0)):
            j = (3 * m + 5 * i) % (K // 32)
            X[m, 32 * j:32 * j + 32] = v
    return X.astype(np.float16)


@pytest.mark.parametrize("tiled", [False, True])
def test_subblock_sums_beyond_binary16(tiled):
    """The min term multiplies each 32-value sub-block sum of X; sums past
    binary16's range must stay finite and exact enough (three binary16 parts)."""
    M, N, K = 12, 100, 2048
    W, _ = inputs(N, K, M, tag=17)
    X = _big_sum_rows(M, K, 17)
    if tiled:
        Y = tiled_pair(W, X, N)[1]
    else:
        Y = run_gpu(W, X)
    assert np.all(np.isfinite(Y))
    _, worst = check(W, X, Y=Y)
    print(f"large sub-block sums (tiled={tiled}) worst |err|/S = {worst:.3e}")


def _cancel_blocks(dmin_bits, n_rows, kb):
    """d = 1, every scale and min 63, every quant 15: the weight's two terms
    are 945 and 63 * dmin; dmin = 15 (0x4B80) makes every weight exactly 0,
    one binary16 step more (0x4B81) makes it -63/128."""
    return _blocks(0x3C00, dmin_bits, 0xFF, 0xFF, n_rows, kb)


@pytest.mark.parametrize("tiled", [False, True])
def test_cancelling_and_near_cancelling_blocks(tiled):
    """Columns 0-15 hold weights that are exactly 0 (the two terms of the
    factored form cancel), 16-31 generated weights, 32-47 weights of -63/128
    made of two terms of about 945. The factored product keeps its error
    within 1e-4 of the size of the two terms (F); generated columns also meet
    1e-4 * sum|w x|."""
    M, K = 12, 1024
    gen, _ = inputs(16, K, M, tag=18)
    W = np.concatenate([_cancel_blocks(0x4B80, 16, K // 256), gen,
                        _cancel_blocks(0x4B81, 16, K // 256)])
    X = synth.activations(18, M, K)
    Y = tiled_pair(W, X, 48)[1] if tiled else run_gpu(W, X)
    y_ref, S = oracle.gemm(W, X)
    F = oracle.factored_size(W, X)
    assert np.all(y_ref[:, :16] == 0) and np.all(S[:, :16] == 0)
    ok, worst_f, nbad = oracle.within_bound(Y, y_ref, F)
    assert ok, f"{nbad} outside 1e-4 * F, worst |err|/F = {worst_f:.3e}"
    ok, worst, nbad = oracle.within_bound(Y[:, 16:32], y_ref[:, 16:32], S[:, 16:32])
    assert ok, f"generated columns: {nbad} outside the bound, worst {worst:.3e}"
    with np.errstate(divide="ignore", invalid="ignore"):
        near = np.max(np.abs(Y[:, 32:] - y_ref[:, 32:]) / S[:, 32:])
    print(f"cancelling (tiled={tiled}): worst |err|/F {worst_f:.3e}, |y| on w=0 "
          f"{np.abs(Y[:, :16]).max():.3e}, near-cancelling |err|/S {near:.3e}")


# --- properties -----------------------------------------------------------------
def test_deterministic_run_to_run():
    W, X = inputs(1000, 5120, 12, tag=12)
    Wt = torch.from_numpy(W).to(DEV)
    Xt = torch.from_numpy(X).to(DEV)
    a = mk.gemm(Wt, Xt).cpu()
    for _ in range(3):
        assert torch.equal(a, mk.gemm(Wt, Xt).cpu())


def test_power_of_two_scaling_exact():
    W, X = inputs(300, 2048, 12, tag=13)
    Wt = torch.from_numpy(W).to(DEV)
    Xt = torch.from_numpy(X).to(DEV)
    y1 = mk.gemm(Wt, Xt).cpu()
    y2 = mk.gemm(Wt, (Xt.float() * 2).half()).cpu()
    assert torch.equal(y2, 2 * y1)


def test_row_permutation():
    W, X = inputs(200, 3072, 12, tag=14)
    perm = np.random.default_rng(1).permutation(12)
    Wt = torch.from_numpy(W).to(DEV)
    y = mk.gemm(Wt, torch.from_numpy(X).to(DEV)).cpu()
    yp = mk.gemm(Wt, torch.from_numpy(np.ascontiguousarray(X[perm])).to(DEV)).cpu()
    assert torch.equal(yp, y[perm])


def test_explicit_workspace_matches_owned():
    W, X = inputs(700, 17408 // 4, 12, tag=15)
    Wt = torch.from_numpy(W).to(DEV)
    Xt = torch.from_numpy(X).to(DEV)
    nbytes = mk.gemm_workspace_bytes(12, 700, 17408 // 4)
    ws = torch.zeros(max(nbytes, 16), dtype=torch.uint8, device=DEV)
    a = mk.gemm(Wt, Xt).cpu()
    b = mk.gemm(Wt, Xt, workspace=ws).cpu()
    assert torch.equal(a, b)


def test_misaligned_pointer_rejected():
    W, X = inputs(16, 256, 1, tag=16)
    Wt = torch.from_numpy(W).to(DEV)
    Xbig = torch.zeros(1, 256 + 1, dtype=torch.float16, device=DEV)
    Xmis = Xbig.view(-1)[1:257].view(1, 256)      # 2-byte offset
    with pytest.raises(mk.MkError) as e:
        mk.gemm(Wt, Xmis)
    assert e.value.code == mk.MK_EALIGN


# --- the tile-record path (mk_q4k_gemm_tiled) ------------------------------------
def tiled_pair(W_np, X_np, N):
    W = torch.from_numpy(np.ascontiguousarray(W_np)).to(DEV)
    X = torch.from_numpy(np.ascontiguousarray(X_np)).to(DEV)
    Wt = mk.repack(W, N, X_np.shape[1])
    y_rows = mk.gemm(W, X)
    y_tiles = mk.gemm_tiled(Wt, X, N)
    torch.cuda.synchronize()
    return y_rows.cpu().numpy(), y_tiles.cpu().numpy()


@pytest.mark.parametrize("M,N,K", [
    (1, 256, 1024), (12, 333, 2048), (16, 17408 // 8, 5120), (33, 100, 1536), (64, 257, 1024),
    (5, 5120 // 4, 17408),
])
def test_tiled_bitwise_equal_to_rows_and_in_bound(M, N, K):
    W, X = inputs(N, K, M, tag=40 + M)
    y_rows, y_tiles = tiled_pair(W, X, N)
    assert np.array_equal(y_rows.view(np.uint32), y_tiles.view(np.uint32))
    check(W, X, Y=y_tiles)


def test_tiled_gate_up_m12_sampled():
    N, K, M = 17408, 5120, 12
    W, X = inputs(N, K, M, tag=50)
    _, y = tiled_pair(W, X, N)
    cols = np.unique(np.random.default_rng(5).choice(N, 2048, replace=False))
    check(W, X, cols=cols, Y=y)


def test_tiled_down_m16_sampled():
    N, K, M = 5120, 17408, 16
    W, X = inputs(N, K, M, tag=51)
    _, y = tiled_pair(W, X, N)
    cols = np.unique(np.concatenate([np.random.default_rng(6).choice(N, 1024, replace=False),
                                     [0, N - 1]]))
    check(W, X, cols=cols, Y=y)


@pytest.mark.parametrize("N,K", [(1, 256), (333, 2048), (5120, 17408)])
def test_repack_column_sums(N, K):
    """The fp32 sums of every output column's dequantized weights that follow
    the tile records: each within one fp32 rounding of the exact float64 sum,
    and zero on the padding columns of the last tile."""
    W, _ = inputs(N, K, 1, tag=70 + N % 7)
    Wt = mk.repack(torch.from_numpy(np.ascontiguousarray(W)).to(DEV), N, K)
    torch.cuda.synchronize()
    nt = (N + 15) // 16
    raw = Wt.cpu().numpy()
    cs = raw[raw.size - nt * 16 * 4:].view(np.float32).astype(np.float64)
    deq = oracle.dequant_rows(W, K)
    ref = deq.sum(axis=1)
    # one fp32 rounding, plus the float64 summation-order slack of both sides
    tol = np.spacing(np.abs(ref).astype(np.float32)) + 1e-13 * np.abs(deq).sum(axis=1)
    assert np.all(np.abs(cs[:N] - ref) <= tol)
    assert np.all(cs[N:] == 0.0)


def test_interleaved_shapes_keep_the_workspace_consistent():
    """Calls of different shapes (each splitting K) share the library
    workspace; every call must leave its counters ready for the next one."""
    a = inputs(300, 17408, 12, tag=60)
    b = inputs(500, 8192, 4, tag=61)
    ya = run_gpu(*a)
    yb = run_gpu(*b)
    ya2 = run_gpu(*a)
    yb2 = run_gpu(*b)
    assert np.array_equal(ya, ya2) and np.array_equal(yb, yb2)
    check(*a, Y=ya)
    check(*b, Y=yb)


# --- batch invariance: a row's result does not depend on the rows beside it ----
@pytest.mark.parametrize("N,K", [(333, 2048), (17408 // 8, 5120), (5120 // 4, 17408)])
def test_rows_bit_identical_alone_or_stacked(N, K):
    """The K split is chosen for 64 rows whatever M is, so every output is
    summed in the same order: the first M' rows of a 64-row call, and single
    rows called alone, match it bit for bit (row and tile-record layouts)."""
    W, X = inputs(N, K, 64, tag=80)
    Wd = torch.from_numpy(W).to(DEV)
    Xd = torch.from_numpy(X).to(DEV)
    Wt = mk.repack(Wd, N, K)
    full = mk.gemm(Wd, Xd)
    full_t = mk.gemm_tiled(Wt, Xd, N)
    torch.cuda.synchronize()
    assert torch.equal(full, full_t)
    for m in (1, 5, 12, 16, 33):
        assert torch.equal(mk.gemm(Wd, Xd[:m].contiguous()), full[:m]), m
        assert torch.equal(mk.gemm_tiled(Wt, Xd[:m].contiguous(), N), full[:m]), m
    for r in (0, 13, 40, 63):
        assert torch.equal(mk.gemm(Wd, Xd[r:r + 1].contiguous()), full[r:r + 1]), r
