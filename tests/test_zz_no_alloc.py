"""mk_q4k_gemm_noalloc (the GEMM entry point that allocates nothing: its
K-split partial sums live in the library's static per-GPU scratch array)
against mk_q4k_gemm, which keeps them in a library-owned allocation: the
same kernels and plan, so the results must agree bit for bit, on two calls in
a row where the second is smaller, and both against the fp64 oracle. Every
call goes through the C ABI."""
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


def _inputs(N, K, M, tag):
    W = synth.q4k_matrix(synth.key(0, synth.TAG_WEIGHT, tag, N * 100003 + K), N, K)
    X = synth.activations(tag, M, K)
    return W, X


def test_noalloc_matches_gemm_on_two_calls_second_smaller():
    big = _inputs(17408, 5120, 12, 91)       # 5.3 MiB of partials
    small = _inputs(333, 2048, 4, 92)        # fewer, at other offsets
    outs = []
    for W, X in (big, small):
        Wd, Xd = torch.from_numpy(W).to(DEV), torch.from_numpy(X).to(DEV)
        y_na = mk.gemm_noalloc(Wd, Xd)
        torch.cuda.synchronize()
        y_ref = mk.gemm(Wd, Xd)
        torch.cuda.synchronize()
        assert torch.equal(y_na, y_ref), (W.shape, X.shape)
        outs.append(y_na.cpu().numpy())
    # against the oracle: every column of the small call, sampled columns of the big one
    cols = np.unique(np.concatenate([np.random.default_rng(9).choice(17408, 1500, replace=False),
                                     [0, 17407]]))
    y_ref, S = oracle.gemm(big[0][cols], big[1])
    ok, worst, nbad = oracle.within_bound(outs[0][:, cols].astype(np.float64), y_ref, S)
    assert ok, f"big: {nbad} outside the bound, worst {worst:.3e}"
    y_ref, S = oracle.gemm(*small)
    ok, worst2, nbad = oracle.within_bound(outs[1].astype(np.float64), y_ref, S)
    assert ok, f"small: {nbad} outside the bound, worst {worst2:.3e}"
    print(f"noalloc: bit-identical to mk_q4k_gemm; worst |err|/S {max(worst, worst2):.3e}")


def test_noalloc_rejects_shapes_beyond_its_scratch():
    """64 rows of a 34816 x 5120 matrix need 42.5 MiB of partials, more than
    the 24 MiB array: MK_EWORKSPACE, and Y is left untouched."""
    N, K, M = 34816, 5120, 64
    W = torch.zeros((N, K // 256 * 144), dtype=torch.uint8, device=DEV)
    X = torch.zeros((M, K), dtype=torch.float16, device=DEV)
    Y = torch.full((M, N), 7.0, dtype=torch.float32, device=DEV)
    with pytest.raises(mk.MkError) as e:
        mk.gemm_noalloc(W, X, out=Y)
    assert e.value.code == mk.MK_EWORKSPACE
    torch.cuda.synchronize()
    assert bool(torch.all(Y == 7.0))
