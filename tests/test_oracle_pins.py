"""Pins of the CPU oracle to facts outside itself (CPU only).

Every check here compares the oracle with something the pages, the public
Q4_K block definition or plain mathematics fixes: hand-worked bytes and
weights (tests/golden/), exhaustive round trips, unit vectors, closed forms,
and library routines for the pieces that have one (numpy's binary16 decoding
and rounding, numpy's float64/int64 matrix products). The pieces are chosen so
that a dropped term, a wrong sign, a wrong nibble or bit index or a transposed
operand fails at least one of them.
"""
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def make_block(d_bits=0, dmin_bits=0, scales=None, qs=None):
    """Assemble 144 block bytes from raw fields (no arithmetic of the method)."""
    b = bytearray(144)
    b[0:2] = int(d_bits).to_bytes(2, "little")
    b[2:4] = int(dmin_bits).to_bytes(2, "little")
    if scales is not None:
        b[4:16] = bytes(scales)
    if qs is not None:
        b[16:144] = bytes(qs)
    return bytes(b)


def pack_scales_from_spec(sc, mn):
    """Inverse of the 12-byte scale/min packing, written from the layout rule:
    sub-blocks 0..3 sit in the low 6 bits of bytes 0..3 (scale) and 4..7 (min);
    sub-blocks 4..7 put their low 4 bits in bytes 8..11 (scale low nibble, min
    high nibble) and their top 2 bits in bits 6..7 of bytes 0..3 (scale) and
    4..7 (min)."""
    s = [0] * 12
    for j in range(4):
        s[j] = sc[j] & 63
        s[j + 4] = mn[j] & 63
    for j in range(4, 8):
        s[j + 4] = (sc[j] & 15) | ((mn[j] & 15) << 4)
        s[j - 4] |= (sc[j] >> 4) << 6
        s[j] |= (mn[j] >> 4) << 6
    return bytes(s)


# ---------------------------------------------------------------- binary16

def test_f16_decode_exhaustive_vs_numpy():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.f16_to_f64(bits)
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    # signed zeros and subnormal extremes by hand
    assert ours[0x0001] == 2.0 ** -24
    assert ours[0x03FF] == 1023 * 2.0 ** -24
    assert ours[0x0400] == 2.0 ** -14
    assert ours[0x3C00] == 1.0 and ours[0x7BFF] == 65504.0
    assert np.isinf(ours[0x7C00]) and np.signbit(ours[0x8000])


def test_f64_to_f16_vs_numpy():
    rng = np.random.default_rng(1)
    v = np.concatenate([
        rng.standard_normal(200000),
        rng.standard_normal(50000) * 1e-5,          # subnormal range
        rng.standard_normal(50000) * 3e4,           # near overflow
        np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, -65520.0, 1e9, 2.0 ** -25,
                  3 * 2.0 ** -25, 2.0 ** -24 * 1.5, 2.0 ** -14 - 2.0 ** -26]),
    ])
    # exact ties: midpoints between consecutive binary16 values
    h = np.arange(0x0000, 0x7BFF, 7, dtype=np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).view(np.float16).astype(np.float64)
    v = np.concatenate([v, (lo + hi) / 2, -(lo + hi) / 2])
    ours = oracle.f64_to_f16(v)
    ref = v.astype(np.float16).view(np.uint16)
    assert np.array_equal(ours, ref)


# ------------------------------------------------------- scale/min packing

def _golden_scale_lines():
    with open(os.path.join(GOLDEN, "q4k_scale_bytes.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            b, sc, mn = (p.split() for p in line.split("|"))
            yield bytes(int(x, 16) for x in b), [int(x) for x in sc], [int(x) for x in mn]


def test_scale_bytes_golden():
    n = 0
    for b, sc, mn in _golden_scale_lines():
        got_sc, got_mn = oracle.unpack_scales(b)
        assert list(got_sc) == sc, b.hex()
        assert list(got_mn) == mn, b.hex()
        # the spec-side packer is the inverse on these hand-worked lines
        assert pack_scales_from_spec(sc, mn) == b
        n += 1
    assert n >= 7


def test_scale_roundtrip_exhaustive():
    # every (sub-block j, scale, min) in 8 x 64 x 64, other sub-blocks zero
    for j in range(8):
        for s in range(64):
            for m in range(0, 64, 1):
                sc = [0] * 8
                mn = [0] * 8
                sc[j] = s
                mn[j] = m
                got_sc, got_mn = oracle.unpack_scales(pack_scales_from_spec(sc, mn))
                if list(got_sc) != sc or list(got_mn) != mn:
                    pytest.fail(f"j={j} sc={s} m={m}: {got_sc} {got_mn}")


def test_scale_roundtrip_random_full():
    rng = np.random.default_rng(7)
    for _ in range(2000):
        sc = [int(x) for x in rng.integers(0, 64, 8)]
        mn = [int(x) for x in rng.integers(0, 64, 8)]
        got_sc, got_mn = oracle.unpack_scales(pack_scales_from_spec(sc, mn))
        assert list(got_sc) == sc and list(got_mn) == mn


# ------------------------------------------------------------ nibble order

def test_single_nibble_unit_vectors():
    """d = 1, dmin = 0, every scale 1, exactly one quant set to 1: the block
    dequantizes to the unit vector e_t. The nibble is placed by the layout
    rule: weight t = 64c + 32h + i lives in quant byte 32c + i, low nibble for
    h = 0 and high nibble for h = 1."""
    ones = pack_scales_from_spec([1] * 8, [0] * 8)
    rows = []
    for t in range(256):
        c, r = divmod(t, 64)
        h, i = divmod(r, 32)
        qs = bytearray(128)
        qs[32 * c + i] = 0x01 if h == 0 else 0x10
        rows.append(make_block(0x3C00, 0x0000, ones, qs))
    W = np.frombuffer(b"".join(rows), dtype=np.uint8).reshape(256, 144)
    w = oracle.dequant_rows(W, 256)
    assert np.array_equal(w, np.eye(256))


# ---------------------------------------------------------- dequant formula

def test_all_zero_block():
    W = np.zeros((3, 4 * 144), dtype=np.uint8)
    w = oracle.dequant_rows(W, 1024)
    assert np.all(w == 0)
    X = synth.activations(0, 5, 1024)
    y, S = oracle.gemm(W, X)
    assert np.all(y == 0) and np.all(S == 0)


def test_max_scale_block():
    # d = dmin = 1, every scale and min 63, every quant 15: w = 63*15 - 63 = 882
    blk = make_block(0x3C00, 0x3C00, pack_scales_from_spec([63] * 8, [63] * 8), [0xFF] * 128)
    assert blk[4:16] == bytes([0xFF] * 12)
    w = oracle.dequant_rows(np.frombuffer(blk, dtype=np.uint8), 256)
    assert np.all(w == 882.0)


def test_min_only_block():
    # all quants 0: w = -dmin * m_j on every weight of sub-block j
    mn = [3, 0, 63, 17, 1, 44, 9, 60]
    blk = make_block(0x3C00, 0x3400, pack_scales_from_spec([5] * 8, mn), [0] * 128)  # dmin=0.25
    w = oracle.dequant_rows(np.frombuffer(blk, dtype=np.uint8), 256)[0]
    for j in range(8):
        assert np.all(w[32 * j:32 * j + 32] == -0.25 * mn[j])


def test_subnormal_d():
    # d = 2^-24 (smallest subnormal), one weight with scale 63 and quant 15
    blk = make_block(0x0001, 0x0000, pack_scales_from_spec([63] * 8, [0] * 8),
                     [0x0F] + [0] * 127)
    w = oracle.dequant_rows(np.frombuffer(blk, dtype=np.uint8), 256)[0]
    assert w[0] == 63 * 15 * 2.0 ** -24
    assert np.count_nonzero(w) == 1


def test_handbuilt_block_golden():
    fields = {"qs": []}
    ws = []
    with open(os.path.join(GOLDEN, "q4k_block_handbuilt.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            k, *rest = line.split()
            if k == "qs":
                fields["qs"].append((int(rest[0]), int(rest[1], 16)))
            elif k == "w":
                ws.append((int(rest[0]), float(rest[1])))
            elif k == "scales":
                fields[k] = bytes(int(x, 16) for x in rest)
            else:
                fields[k] = int(rest[0], 16)
    qs = bytearray(128)
    for off, val in fields["qs"]:
        qs[off] = val
    blk = make_block(fields["d"], fields["dmin"], fields["scales"], qs)
    w = oracle.dequant_rows(np.frombuffer(blk, dtype=np.uint8), 256)[0]
    assert len(ws) >= 9
    for t, val in ws:
        assert w[t] == val, (t, w[t], val)


# ------------------------------------------------------------------- matmul

def test_constant_scale_closed_form():
    """With d, dmin, sc, m the same in every block, W = d*sc*Q - dmin*m*J, so
    Y = d*sc*(X Q^T) - dmin*m*rowsum(X) 1^T with X Q^T an exact integer-weight
    product (checked with int64 arithmetic on the scaled fp16 inputs). Rows
    and columns differ in count so a transposed operand cannot pass."""
    rng = np.random.default_rng(3)
    M, N, K = 5, 37, 768
    d_bits, dmin_bits = 0x1E00, 0x1A00          # 0.005859375 and 0.0029296875
    sc, m = 41, 13
    scales = pack_scales_from_spec([sc] * 8, [m] * 8)
    Q = rng.integers(0, 16, size=(N, K))
    rows = []
    for n in range(N):
        blocks = []
        for kb in range(K // 256):
            q = Q[n, 256 * kb:256 * kb + 256]
            qs = bytearray(128)
            for c in range(4):
                for i in range(32):
                    qs[32 * c + i] = int(q[64 * c + i]) | (int(q[64 * c + 32 + i]) << 4)
            blocks.append(make_block(d_bits, dmin_bits, scales, qs))
        rows.append(b"".join(blocks))
    W = np.frombuffer(b"".join(rows), dtype=np.uint8).reshape(N, -1)
    X = (rng.standard_normal((M, K))).astype(np.float16)
    y, S = oracle.gemm(W, X)

    d = float(np.array([d_bits], dtype=np.uint16).view(np.float16)[0])
    dmin = float(np.array([dmin_bits], dtype=np.uint16).view(np.float16)[0])
    # every fp16 value is an integer multiple of 2^-24: exact int64 products
    xi = (X.astype(np.float64) * 2.0 ** 24).astype(np.int64)
    xq = xi @ Q.T.astype(np.int64)               # exact
    xs = xi.sum(axis=1, keepdims=True)           # exact
    y_cf = d * sc * (xq.astype(np.float64) * 2.0 ** -24) - dmin * m * (xs * 2.0 ** -24)
    assert np.allclose(y, y_cf, rtol=0, atol=1e-9 * np.abs(S).max())
    # and tighter, per element, against the error scale
    assert np.all(np.abs(y - y_cf) <= 1e-12 * S + 1e-300)


def test_gemm_vs_numpy_matmul_and_abs():
    rng = np.random.default_rng(11)
    M, N, K = 7, 53, 1280
    W = synth.q4k_matrix(synth.key(5, 9), N, K)
    X = synth.f16_normal(synth.key(5, 10), M * K).reshape(M, K)
    y, S = oracle.gemm(W, X)
    w = oracle.dequant_rows(W, K)
    x = X.astype(np.float64)
    y_np = x @ w.T
    S_np = np.abs(x) @ np.abs(w).T
    assert np.all(np.abs(y - y_np) <= 1e-12 * S)
    assert np.allclose(S, S_np, rtol=1e-12, atol=0)
    # a transposed or row-swapped result would not match
    assert y.shape == (M, N)
    del rng


def test_oracle_error_far_below_tolerance():
    """The oracle's own rounding is ~K * 2^-53 * S, far below the 1e-4 * S bound:
    compare against an exact rational evaluation on a small case."""
    from fractions import Fraction
    M, N, K = 2, 3, 512
    W = synth.q4k_matrix(synth.key(8, 1), N, K)
    X = synth.f16_normal(synth.key(8, 2), M * K).reshape(M, K)
    y, S = oracle.gemm(W, X)
    w = oracle.dequant_rows(W, K)              # exact values (checked above)
    x = X.astype(np.float64)
    for m in range(M):
        for n in range(N):
            exact = sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(x[m], w[n]))
            assert abs(Fraction(float(y[m, n])) - exact) <= Fraction(1, 10 ** 12) * Fraction(float(S[m, n]))


# ---------------------------------------------------- transform and bounds

def test_standardize_moments_and_small_case():
    v = np.array([[1.0, 2.0, 3.0, 4.0], [10.0, 10.0, 10.0, 10.0]])
    t = oracle.standardize(v, eps=1e-6)
    # row 0: mean 2.5, population variance 1.25
    assert np.allclose(t[0], (v[0] - 2.5) / np.sqrt(1.25 + 1e-6), rtol=1e-15, atol=0)
    # a constant row maps to exact zeros
    assert np.all(t[1] == 0.0)
    rng = np.random.default_rng(2)
    v = rng.standard_normal((6, 5000)) * 30 + 7
    t = oracle.standardize(v, eps=1e-6)
    assert np.allclose(t.mean(axis=1), 0, atol=1e-12)
    var = v.var(axis=1)
    assert np.allclose(t.var(axis=1), var / (var + 1e-6), rtol=1e-12)


def test_row_moments_closed_form_and_standardize():
    v = np.array([[1.0, 2.0, 3.0, 4.0], [10.0, 10.0, 10.0, 10.0], [-2.0, 2.0, -2.0, 2.0]])
    mean, inv = oracle.row_moments(v, eps=1e-6)
    # population variance: 1.25, 0 and 4
    assert list(mean) == [2.5, 10.0, 0.0]
    assert np.allclose(inv, 1.0 / np.sqrt(np.array([1.25, 0.0, 4.0]) + 1e-6), rtol=1e-15, atol=0)
    t = oracle.standardize(v, eps=1e-6)
    assert np.array_equal(t, (v - mean[:, None]) * inv[:, None])
    # binary16 input is taken at its exact values
    x = np.array([[0.5, -1.5, 3.0, 65504.0]], dtype=np.float16)
    m16, _ = oracle.row_moments(x)
    assert m16[0] == (0.5 - 1.5 + 3.0 + 65504.0) / 4


def test_factored_size_hand_worked_block():
    """d = 0.5, dmin = 0.25, every scale 3, min 5 and quant 6: each weight's
    two terms are d*sc*q = 9 and dmin*m = 1.25 (w = 7.75). Against a row of
    alternating 1, -2 (sum |x| = 384): F = 10.25 * 384 = 3936 and S = 7.75 *
    384 = 2976; with a row mean of 0.5 and scale r = 2,
    F = 2 * (3936 + |0.5 * 7.75 * 256|) = 9856."""
    blk = make_block(0x3800, 0x3400, pack_scales_from_spec([3] * 8, [5] * 8), [0x66] * 128)
    W = np.frombuffer(blk, dtype=np.uint8).reshape(1, 144)
    X = np.tile(np.array([1.0, -2.0], dtype=np.float16), 128).reshape(1, 256)
    F = oracle.factored_size(W, X)
    _, S = oracle.gemm(W, X)
    assert F[0, 0] == 3936.0 and S[0, 0] == 2976.0
    F2 = oracle.factored_size(W, X, mean=np.array([0.5]), r=np.array([2.0]))
    assert F2[0, 0] == 9856.0


def test_factored_size_cancelling_block():
    """d = 1, sc = 63, q = 15, dmin = 15, m = 63: the two terms are both 945,
    so every weight is 0 (S = 0) while F = 1890 * sum |x|."""
    blk = make_block(0x3C00, 0x4B80, pack_scales_from_spec([63] * 8, [63] * 8), [0xFF] * 128)
    W = np.frombuffer(blk * 2, dtype=np.uint8).reshape(1, 288)
    X = synth.activations(21, 3, 512)
    y, S = oracle.gemm(W, X)
    assert np.all(y == 0) and np.all(S == 0)
    F = oracle.factored_size(W, X)
    assert np.array_equal(F[:, 0], 1890.0 * np.abs(X.astype(np.float64)).sum(axis=1))


def test_factored_size_equals_s_without_opposite_terms_and_bounds_it():
    """Where one of a weight's two terms is 0 (dmin = 0, or q = 0) |w| is the
    sum of the terms' sizes, so F and S are the same sums of the same
    products; on generated weights F >= S (|w| <= |d sc q| + |dmin m|)."""
    N, K, M = 23, 768, 4
    W = synth.q4k_matrix(synth.key(22, 1), N, K)
    X = synth.activations(22, M, K)
    Wb = W.copy().reshape(-1, 144)
    Wb[:, 2:4] = 0                      # dmin = 0
    W0 = Wb.reshape(N, -1)
    assert np.array_equal(oracle.factored_size(W0, X), oracle.gemm(W0, X)[1])
    Wq = W.copy().reshape(-1, 144)
    Wq[:, 16:] = 0                      # q = 0: w = -dmin m
    Wq = Wq.reshape(N, -1)
    assert np.array_equal(oracle.factored_size(Wq, X), oracle.gemm(Wq, X)[1])
    F = oracle.factored_size(W, X)
    S = oracle.gemm(W, X)[1]
    assert np.all(F >= S) and np.any(F > S)


def test_gemm_std_shift_and_scale_invariance():
    """Standardizing the input makes the product independent of a per-row
    offset and of a per-row positive scale (exactly, up to the eps term). The
    inputs sit on a coarse grid so that shifted and doubled copies are exact
    in binary16; a dropped mean, a wrong sign or a missing 1/sigma breaks it."""
    M, N, K = 3, 17, 768
    W = synth.q4k_matrix(synth.key(12, 1), N, K)
    rng = np.random.default_rng(12)
    base = rng.integers(-64, 65, size=(M, K)).astype(np.float64) / 16.0
    X = base.astype(np.float16)
    y, S = oracle.gemm_std(W, X)
    for shift, scale in ((3.0, 1.0), (-5.5, 1.0), (0.0, 2.0), (1.25, 4.0)):
        X2 = ((base + shift) * scale).astype(np.float16)
        assert np.array_equal(X2.astype(np.float64), (base + shift) * scale)  # exact
        y2, S2 = oracle.gemm_std(W, X2)
        var = base.var(axis=1, keepdims=True)
        # eps breaks exact scale invariance by a factor sqrt((var + eps) / (s^2 var + eps))
        f = np.sqrt((var + 1e-6) / (scale * scale * var + 1e-6)) * scale
        assert np.all(np.abs(y2 - y * f) <= 1e-12 * S2), (shift, scale)
        assert np.allclose(S2, S * f, rtol=1e-12), (shift, scale)


def test_gemm_std_constant_row_is_zero_and_matches_numpy():
    M, N, K = 4, 29, 1024
    W = synth.q4k_matrix(synth.key(13, 1), N, K)
    X = synth.f16_normal(synth.key(13, 2), M * K).reshape(M, K).copy()
    X[2, :] = np.float16(3.5)                      # constant row: variance 0
    y, S = oracle.gemm_std(W, X)
    assert np.all(y[2] == 0.0) and np.all(S[2] == 0.0)
    # numpy: standardize the decoded input, then a float64 matmul with the
    # dequantized weights
    x = X.astype(np.float64)
    mu = x.mean(axis=1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=1, keepdims=True)
    t = (x - mu) / np.sqrt(var + 1e-6)
    w = oracle.dequant_rows(W, K)
    y_np = t @ w.T
    S_np = np.abs(t) @ np.abs(w).T
    assert np.all(np.abs(y - y_np) <= 1e-12 * S_np + 1e-300)
    assert np.allclose(S, S_np, rtol=1e-12, atol=1e-300)


def test_gemm_std_alternating_row_closed_form():
    """A row of +s, -s, +s, ... has mean 0 and variance s^2: the standardized
    product is s / sqrt(s^2 + eps) times the plain product of the +-1 row
    (the plain oracle GEMM, pinned above)."""
    M, N, K = 2, 11, 512
    W = synth.q4k_matrix(synth.key(14, 1), N, K)
    z = np.where(np.arange(K) % 2 == 0, 1.0, -1.0)
    for s in (0.5, 3.0, 1e-3):
        X = np.stack([z * s, -z * s]).astype(np.float16)
        sv = float(X.astype(np.float64)[0, 0])
        y, S = oracle.gemm_std(W, X)
        yz, Sz = oracle.gemm(W, np.stack([z, -z]).astype(np.float16))
        f = abs(sv) / np.sqrt(sv * sv + 1e-6)
        assert np.all(np.abs(y - f * yz) <= 1e-12 * S + 1e-300), s
        assert np.allclose(S, f * Sz, rtol=1e-12), s


# --- the residual walk: RMSNorm scale, scaled product, SiLU --------------------
def test_rms_inv_closed_forms():
    """Constant rows c: 1/sqrt(c^2 + eps); alternating +-a: 1/sqrt(a^2 + eps);
    a (3, 4, 3, 4, ...) row: mean square 12.5. A dropped square, a missing
    1/N or eps outside the root breaks one of them."""
    h = np.array([[2.0] * 8, [-3.0] * 8, [1.5, -1.5] * 4, [3.0, 4.0] * 4, [0.0] * 8])
    for eps in (0.0, 1e-6, 0.25):
        r = oracle.rms_inv(h, eps)
        want = 1.0 / np.sqrt(np.array([4.0, 9.0, 2.25, 12.5, 0.0]) + eps)
        if eps == 0.0:
            assert np.allclose(r[:4], want[:4], rtol=1e-15) and np.isinf(r[4])
        else:
            assert np.allclose(r, want, rtol=1e-15)


def test_rms_inv_matches_numpy_and_scales():
    h = synth.normals(synth.key(20, 1), 6 * 1000).reshape(6, 1000) * 7.0
    r = oracle.rms_inv(h, 1e-6)
    assert np.allclose(r, 1.0 / np.sqrt((h * h).mean(axis=1) + 1e-6), rtol=1e-13)
    # without eps the scale is exactly inverse-proportional to a power-of-two factor
    assert np.array_equal(oracle.rms_inv(h * 8.0, 0.0) * 8.0, oracle.rms_inv(h, 0.0))


def test_gemm_rms_reduces_to_gemm_and_scales_exactly():
    """At unit scale the normed product is the plain oracle GEMM bit for bit;
    a power-of-two row scale scales y and S exactly; a general scale agrees
    with r * gemm to rounding."""
    M, N, K = 3, 23, 768
    W = synth.q4k_matrix(synth.key(21, 1), N, K)
    X = synth.f16_normal(synth.key(21, 2), M * K).reshape(M, K)
    y0, S0 = oracle.gemm(W, X)
    y1, S1 = oracle.gemm_rms(W, X, np.ones(M))
    assert np.array_equal(y1, y0) and np.array_equal(S1, S0)
    r2 = np.array([0.125, 4.0, 2.0 ** -20])
    y2, S2 = oracle.gemm_rms(W, X, r2)
    assert np.array_equal(y2, y0 * r2[:, None]) and np.array_equal(S2, S0 * r2[:, None])
    r3 = np.array([0.3, 1.7, 0.05])
    y3, S3 = oracle.gemm_rms(W, X, r3)
    assert np.all(np.abs(y3 - y0 * r3[:, None]) <= 1e-13 * S3)
    # numpy: scale the decoded input, float64 matmul with the dequantized weights
    t = X.astype(np.float64) * r3[:, None]
    w = oracle.dequant_rows(W, K)
    assert np.all(np.abs(y3 - t @ w.T) <= 1e-12 * S3)


def test_silu_identities_and_values():
    """silu(v) - silu(-v) = v; silu(0) = 0; silu(1) = e / (1 + e); silu(v) -> v
    for large v and -> 0 for very negative v; numpy's v / (1 + exp(-v))."""
    v = synth.normals(synth.key(22, 1), 2000) * 6.0
    a, b = oracle.silu(v), oracle.silu(-v)
    assert np.allclose(a - b, v, rtol=1e-14, atol=1e-15)
    assert oracle.silu(np.array([0.0]))[0] == 0.0
    e = np.e
    assert abs(oracle.silu(np.array([1.0]))[0] - e / (1.0 + e)) <= 1e-16
    big = oracle.silu(np.array([40.0, -40.0]))
    assert big[0] == 40.0 and 0.0 > big[1] > -1e-15
    assert np.allclose(a, v / (1.0 + np.exp(-v)), rtol=1e-15, atol=1e-300)


def test_centered_generator_gives_zero_mean_weights():
    """The centred blocks of the residual walk: scales 1..4, mins 15*scale,
    dmin about d/2, so each sub-block is d*sc*(q - 7.5) up to the rounding of
    dmin (checked through the pinned block decoder)."""
    W = synth.q4k_rows_centered(synth.key(23, 1), 1024, 0, 32)
    for row in W.reshape(-1, 144)[:64]:
        d, dmin, sc, mn, q = oracle.decode_block(row)
        assert np.all((sc >= 1) & (sc <= 4)) and np.array_equal(mn, 15 * sc)
        assert abs(dmin - d / 2) <= 2.0 ** -11 * d + 2.0 ** -24  # two binary16 roundings
    w = oracle.dequant_rows(W, 1024)
    assert abs(w.mean()) < 0.01 * w.std()


def test_within_bound_rule():
    y_ref = np.array([1.0, 0.0, -2.0])
    S = np.array([10.0, 0.0, 4.0])
    assert oracle.within_bound(np.array([1.0009, 0.0, -2.0004]), y_ref, S)[0]
    assert not oracle.within_bound(np.array([1.0011, 0.0, -2.0]), y_ref, S)[0]
    assert not oracle.within_bound(np.array([1.0, 1e-30, -2.0]), y_ref, S)[0]
    assert not oracle.within_bound(np.array([np.nan, 0.0, -2.0]), y_ref, S)[0]


def test_generated_fields_are_uniform():
    """Decoded fields of generated blocks cover their whole range uniformly: a
    decoder that drops the top scale bits or mixes up nibbles would not."""
    W = synth.q4k_matrix(synth.key(0, 77), 64, 256 * 16)       # 1024 blocks
    sc_all, mn_all, q_all, d_all = [], [], [], []
    for blk in W.reshape(-1, 144):
        d, dmin, sc, mn, q = oracle.decode_block(blk.tobytes())
        sc_all.append(sc)
        mn_all.append(mn)
        q_all.append(q)
        d_all += [d, dmin]
    for vals, hi in ((np.concatenate(sc_all), 64), (np.concatenate(mn_all), 64),
                     (np.concatenate(q_all), 16)):
        counts = np.bincount(vals, minlength=hi)
        assert counts.size == hi
        exp = vals.size / hi
        chi2 = float(((counts - exp) ** 2 / exp).sum())
        assert chi2 < hi + 6 * np.sqrt(2 * hi), chi2
    d_all = np.array(d_all)
    assert np.all(d_all >= 0)
    # E|z| * 1e-3 = sqrt(2/pi) * 1e-3
    assert abs(d_all.mean() - np.sqrt(2 / np.pi) * 1e-3) < 5e-5


# --- decode attention over the paged q8_0 pool ---------------------------------
def _page(kq=None, ks=None, vq=None, vs=None):
    """Assemble a 4352-byte page-head from fields [16 tokens][128 dims] (quants)
    and [16 tokens][4 blocks] (scales), each placed at the offset the pool
    layout gives it."""
    b = np.zeros(4352, dtype=np.uint8)
    for t in range(16):
        for d in range(128):
            blk = d // 32
            if kq is not None:
                b[1024 * (blk // 2) + 16 * (16 * ((d % 32) // 8) + t) + 8 * (blk % 2) + d % 8] = \
                    np.int8(kq[t][d]).view(np.uint8)
            if vq is not None:
                b[1024 * (2 + d // 64) + 16 * (16 * (t // 4) + d % 16) + 4 * ((d // 16) % 4) + t % 4] = \
                    np.int8(vq[t][d]).view(np.uint8)
        for blk in range(4):
            at = 4096 + 64 * (t // 4) + 2 * (4 * (t % 4) + blk)
            if ks is not None:
                b[at:at + 2] = np.array([ks[t][blk]], dtype=np.float16).view(np.uint8)
            if vs is not None:
                b[at + 32:at + 34] = np.array([vs[t][blk]], dtype=np.float16).view(np.uint8)
    return b


def test_q8_page_layout_raw_bytes():
    """Raw bytes at offsets worked out by hand from the layout: K quant
    (token 3, dim 40) lives at 16 * (16 * 1 + 3) + 8 = 312 with its scale
    (token 3, block 1) at 4096 + 2 * 13 = 4122; V quant (token 6, dim 77) at
    1024 * 3 + 16 * (16 * 1 + 13) + 4 * 0 + 2 = 3538 with its scale (token 6,
    block 2) at 4096 + 64 + 32 + 2 * 10 = 4212."""
    b = np.zeros(4352, dtype=np.uint8)
    b[312] = np.int8(-7).view(np.uint8)
    b[4122:4124] = np.array([0.5], dtype=np.float16).view(np.uint8)
    b[3538] = np.int8(100).view(np.uint8)
    b[4212:4214] = np.array([0.125], dtype=np.float16).view(np.uint8)
    k, v = oracle.q8_page(b)
    assert k[3, 40] == -3.5 and np.count_nonzero(k) == 1
    assert v[6, 77] == 12.5 and np.count_nonzero(v) == 1


def test_q8_page_decodes_by_hand():
    """Token t, dim d: K = ks[t][d // 32] * kq[t][d]; V likewise. A
    transposed V or a wrong scale block fails."""
    kq = np.zeros((16, 128), dtype=np.int64)
    kq[3, 40] = -7          # token 3, dim 40: block 1
    kq[15, 127] = 127
    ks = np.zeros((16, 4))
    ks[3, 1] = 0.5
    ks[15, 3] = 2.0 ** -10
    vq = np.zeros((16, 128), dtype=np.int64)
    vq[2, 5] = -128
    vs = np.zeros((16, 4))
    vs[2, 0] = 0.25
    k, v = oracle.q8_page(_page(kq, ks, vq, vs))
    want_k = np.zeros((16, 128))
    want_k[3, 40] = -3.5
    want_k[15, 127] = 127 * 2.0 ** -10
    want_v = np.zeros((16, 128))
    want_v[2, 5] = -32.0
    assert np.array_equal(k, want_k) and np.array_equal(v, want_v)


def _page_vscales(ph):
    """[16][4] V scales of a page-head, read from the bytes the layout puts
    them at: 64-byte groups per four tokens at 4096, K scales [token][block]
    then V scales."""
    ph = np.asarray(ph, dtype=np.uint8)
    out = np.empty((16, 4))
    for t in range(16):
        for b in range(4):
            at = 4096 + 64 * (t // 4) + 2 * (4 * (t % 4) + b) + 32
            out[t, b] = ph[at:at + 2].copy().view(np.float16)[0]
    return out


def test_attn_bound_per_element_with_floor():
    """Two tokens: token 0 takes nearly all the weight but its value is 0 in
    dim 1; token 1 has weight p1 = 1 / (1 + e^delta) and value 8 there. The
    bound of dim 1 is p1 * 8 (the only term) plus the floor 2^-80 * the
    largest V scale (0.5): a per-element sum, not the size of the row."""
    kq = np.zeros((16, 128), dtype=np.int64)
    kq[0, 0] = 100
    ks = np.zeros((16, 4))
    ks[0, 0] = 0.5
    vq = np.zeros((16, 128), dtype=np.int64)
    vq[0, 0], vq[1, 1] = 100, 16
    vs = np.zeros((16, 4))
    vs[0, 0] = 0.5
    vs[1, 0] = 0.5
    pool = _one_page_pool(kq, ks, vq, vs)
    Q = np.zeros((1, 1, 128), dtype=np.float16)
    Q[0, 0, 0] = 4.0
    O, S = oracle.attn_decode(Q, pool, np.zeros((1, 1), np.int32), np.zeros(1, np.int32),
                              np.array([2], np.int32), 1)
    delta = 4.0 * 100 * 0.5 / np.sqrt(128.0)
    p1 = 1.0 / (1.0 + np.exp(delta))
    assert np.isclose(O[0, 0, 1], p1 * 8.0, rtol=1e-12, atol=0)
    assert np.isclose(S[0, 0, 1], p1 * 8.0 + 2.0 ** -80 * 0.5, rtol=1e-12, atol=0)
    assert np.isclose(S[0, 0, 0], (1 - p1) * 50.0 + 2.0 ** -80 * 0.5, rtol=1e-12, atol=0)
    assert S[0, 0, 2] == 2.0 ** -80 * 0.5        # no term: the floor alone
    assert O[0, 0, 2] == 0.0


def _one_page_pool(kq, ks, vq, vs):
    return _page(kq, ks, vq, vs).reshape(1, 1, 4352)


def test_attn_single_token_and_equal_keys():
    """One token: O = v_0 exactly. n tokens with equal keys: uniform weights,
    O = mean of v (closed form), whatever the query."""
    rng = np.random.default_rng(30)
    vq = rng.integers(-128, 128, size=(16, 128))
    vs = np.full((16, 4), 0.125)
    kq = np.tile(rng.integers(-128, 128, size=(1, 128)), (16, 1))   # all keys equal
    ks = np.full((16, 4), 0.03125)
    pool = _one_page_pool(kq, ks, vq, vs)
    Q = rng.standard_normal((5, 1, 128)).astype(np.float16)
    table = np.zeros((1, 1), dtype=np.int32)
    lens = np.array([1, 2, 7, 16, 16], dtype=np.int32)
    O, S = oracle.attn_decode(Q, pool, table, np.zeros(5, np.int32), lens, 1)
    v = vq * 0.125
    for r, n in enumerate(lens):
        assert np.allclose(O[r, 0], v[:n].mean(axis=0), rtol=1e-14, atol=1e-14)
        # S: the mean of |v| per dim (equal weights), plus 2^-80 * the V scale
        assert np.allclose(S[r, 0], np.abs(v[:n]).mean(axis=0) + 2.0 ** -80 * 0.125,
                           rtol=1e-14, atol=0)
    assert np.array_equal(O[0, 0], v[0])


def test_attn_two_tokens_closed_form():
    """Two tokens whose scores differ by delta: p_1 = 1 / (1 + exp(-delta))."""
    kq = np.zeros((16, 128), dtype=np.int64)
    kq[0, 0], kq[1, 0] = 10, 30
    ks = np.zeros((16, 4))
    ks[0, 0] = ks[1, 0] = 0.0625
    vq = np.zeros((16, 128), dtype=np.int64)
    vq[0, :] = 8
    vq[1, :] = -24
    vs = np.full((16, 4), 0.5)
    pool = _one_page_pool(kq, ks, vq, vs)
    Q = np.zeros((1, 1, 128), dtype=np.float16)
    Q[0, 0, 0] = 2.0
    O, _ = oracle.attn_decode(Q, pool, np.zeros((1, 1), np.int32), np.zeros(1, np.int32),
                              np.array([2], np.int32), 1)
    delta = 2.0 * (30 - 10) * 0.0625 / np.sqrt(128.0)
    p1 = 1.0 / (1.0 + np.exp(-delta))
    assert np.allclose(O[0, 0], (1 - p1) * 4.0 + p1 * (-12.0), rtol=1e-14)


def test_attn_matches_numpy_with_paging_and_gqa():
    """A shared pool, per-agent page lists, causal row lengths and two query
    heads per KV head, against numpy (dequantized pool, explicit softmax)."""
    n_kv, H = 2, 4
    pool = synth.q8_pool(31, 24, n_kv)
    table, ra, rl = synth.attn_layout(31, [70, 33, 150], 3, 24)
    Q = synth.f16_normal(synth.key(31, 9), 9 * H * 128).reshape(9, H, 128)
    O, S = oracle.attn_decode(Q, pool, table, ra, rl, n_kv)
    for r in range(9):
        a = ra[r]
        for h in range(H):
            kvh = h // (H // n_kv)
            ks, vs = [], []
            for i in range(rl[r]):
                k, v = oracle.q8_page(pool[table[a, i // 16], kvh])
                ks.append(k[i % 16])
                vs.append(v[i % 16])
            K, V = np.array(ks), np.array(vs)
            s = K @ Q[r, h].astype(np.float64) / np.sqrt(128.0)
            p = np.exp(s - s.max())
            p /= p.sum()
            assert np.allclose(O[r, h], p @ V, rtol=1e-12, atol=1e-14), (r, h)
            vsmax = max(np.abs(_page_vscales(pool[table[a, i // 16], kvh])[i % 16]).max()
                        for i in range(rl[r]))
            assert np.allclose(S[r, h], p @ np.abs(V) + 2.0 ** -80 * vsmax, rtol=1e-12,
                               atol=0), (r, h)


# --- Q6_K (GGUF k-quant type 14) -----------------------------------------------
def _q6k_block(d=1.0):
    b = np.zeros(210, dtype=np.uint8)
    b[208:210] = np.array([d], dtype=np.float16).view(np.uint8)
    return b


def test_q6k_single_weights_by_hand():
    """One weight per (half, quarter), its bytes placed by hand: weight 241 is
    half 1, quarter 3, place 17, so its low nibble is the high nibble of
    ql[64 + 32 + 17] = ql[113] and its high bits are bits 6-7 of qh[32 + 17],
    i.e. byte 128 + 49 = 177; its scale is sc[241 // 16] = sc[15], byte 207.
    Every other weight of a run with a nonzero scale is q = 0, i.e. -32."""
    b = _q6k_block(0.5)
    b[113] = 0xA0            # high nibble 10
    b[177] = 0x80            # bits 6-7 = 2
    b[207] = np.int8(-3).view(np.uint8)
    w = oracle.q6k_dequant_rows(b, 256)[0]
    want = np.zeros(256)
    want[240:256] = 0.5 * -3 * -32           # q = 0
    want[241] = 0.5 * -3 * ((10 | 2 << 4) - 32)
    assert np.array_equal(w, want)
    # weight 70: half 0, quarter 2, place 6 -> high nibble of ql[6], bits 4-5 of
    # qh[6] (byte 134), scale sc[4] (byte 196)
    b = _q6k_block(2.0)
    b[6] = 0x3F              # low nibble 15 belongs to weight 6, high nibble 3 to weight 70
    b[134] = 0x30            # bits 4-5 = 3 (weight 70); bits 0-1 = 0 (weight 6)
    b[196] = 1
    b[192] = 7
    w = oracle.q6k_dequant_rows(b, 256)[0]
    want = np.zeros(256)
    want[0:16] = 2.0 * 7 * -32
    want[6] = 2.0 * 7 * (15 - 32)
    want[64:80] = 2.0 * 1 * -32
    want[70] = 2.0 * 1 * ((3 | 3 << 4) - 32)
    assert np.array_equal(w, want)
    # weight 160: half 1, quarter 1, place 0 -> low nibble of ql[64 + 32] =
    # ql[96], bits 2-3 of qh[32] (byte 160), scale sc[10] (byte 202)
    b = _q6k_block(1.0)
    b[96] = 0x05
    b[160] = 0x04            # bits 2-3 = 1
    b[202] = 2
    w = oracle.q6k_dequant_rows(b, 256)[0]
    want = np.zeros(256)
    want[160:176] = 2 * -32.0
    want[160] = 2 * ((5 | 1 << 4) - 32)
    assert np.array_equal(w, want)


def test_q6k_middle_quant_is_zero_and_extremes():
    """q = 32 (low 0, high 2) gives 0 whatever the scales; q = 63 and q = 0
    give 31 and -32 times d * scale."""
    b = _q6k_block(1.0)
    b[128:192] = 0xAA        # every high pair = 2
    b[192:208] = np.arange(1, 17, dtype=np.int8).view(np.uint8)
    assert np.array_equal(oracle.q6k_dequant_rows(b, 256)[0], np.zeros(256))
    b[0:128] = 0xFF
    b[128:192] = 0xFF        # q = 63 everywhere
    w = oracle.q6k_dequant_rows(b, 256)[0]
    assert np.array_equal(w, 31.0 * np.repeat(np.arange(1, 17), 16))
    b[0:192] = 0             # q = 0
    w = oracle.q6k_dequant_rows(b, 256)[0]
    assert np.array_equal(w, -32.0 * np.repeat(np.arange(1, 17), 16))


def test_q6k_gemm_matches_dequant_and_subnormal_d():
    """The GEMM is the plain product of the decoded rows (brute force on a
    tiny case), with a subnormal binary16 d kept exact."""
    import synth
    W = synth.q6k_matrix(synth.key(7, 14, 3, 512), 3, 512)
    W[1, 208:210] = np.array([2.0 ** -20], dtype=np.float16).view(np.uint8)   # subnormal
    X = synth.f16_normal(synth.key(7, 15, 2, 512), 2 * 512).reshape(2, 512)
    w = oracle.q6k_dequant_rows(W, 512)
    assert np.all(np.abs(w[1, :256]) <= 2.0 ** -20 * 128 * 32)
    y, S = oracle.q6k_gemm(W, X)
    xd = X.astype(np.float64)
    for m in range(2):
        for n in range(3):
            terms = [w[n, k] * xd[m, k] for k in range(512)]
            assert abs(y[m, n] - sum(terms)) <= 1e-12 * sum(abs(t) for t in terms)
            assert abs(S[m, n] - sum(abs(t) for t in terms)) <= 1e-12 * S[m, n]


def test_attn_empty_rows_are_the_empty_sum():
    """row_len <= 0: no token to attend to, O = 0 and S = 0 (the empty sum);
    the other rows are computed as usual."""
    import synth
    pool = synth.q8_pool(3, 4, 1)
    table = np.array([[0, 1], [2, 3]], dtype=np.int32)
    Q = synth.f16_normal(synth.key(3, 5, 4, 2), 4 * 2 * 128).reshape(4, 2, 128)
    O, S = oracle.attn_decode(Q, pool, table, np.array([0, 0, 1, 1], dtype=np.int32),
                              np.array([0, -3, 17, 1], dtype=np.int32), 1)
    assert np.all(O[:2] == 0) and np.all(S[:2] == 0)
    assert np.all(S[2:] > 0)


# --- Q6_K matrices of the layer walk: the standardized product ----------------
def test_q6k_gemm_std_shift_and_scale_invariance():
    """As for Q4_K: the Q6_K walk reference depends on the input only through
    its row-standardized form, so a per-row offset and a positive per-row
    scale (exact on a coarse binary16 grid) change it only through eps."""
    M, N, K = 3, 13, 768
    W = synth.q6k_matrix(synth.key(15, 14, N, K), N, K)
    rng = np.random.default_rng(15)
    base = rng.integers(-64, 65, size=(M, K)).astype(np.float64) / 16.0
    y, S = oracle.q6k_gemm_std(W, base.astype(np.float16))
    for shift, scale in ((3.0, 1.0), (-5.5, 1.0), (0.0, 2.0), (1.25, 4.0)):
        X2 = ((base + shift) * scale).astype(np.float16)
        assert np.array_equal(X2.astype(np.float64), (base + shift) * scale)
        y2, S2 = oracle.q6k_gemm_std(W, X2)
        var = base.var(axis=1, keepdims=True)
        f = np.sqrt((var + 1e-6) / (scale * scale * var + 1e-6)) * scale
        assert np.all(np.abs(y2 - y * f) <= 1e-12 * S2), (shift, scale)
        assert np.allclose(S2, S * f, rtol=1e-12), (shift, scale)


def test_q6k_gemm_std_alternating_row_and_constant_row():
    """A row of +s, -s, ... standardizes to +-s / sqrt(s^2 + eps): the product
    is that factor times the plain Q6_K product of the +-1 row (pinned by the
    hand-built blocks above); a constant row standardizes to zeros."""
    M, N, K = 3, 9, 512
    W = synth.q6k_matrix(synth.key(16, 14, N, K), N, K)
    z = np.where(np.arange(K) % 2 == 0, 1.0, -1.0)
    for s in (0.5, 3.0, 1e-3):
        X = np.stack([z * s, -z * s, np.full(K, 2.5)]).astype(np.float16)
        sv = float(X.astype(np.float64)[0, 0])
        y, S = oracle.q6k_gemm_std(W, X)
        yz, Sz = oracle.q6k_gemm(W, np.stack([z, -z, np.zeros(K)]).astype(np.float16))
        f = abs(sv) / np.sqrt(sv * sv + 1e-6)
        assert np.all(np.abs(y[:2] - f * yz[:2]) <= 1e-12 * S[:2] + 1e-300), s
        assert np.allclose(S[:2], f * Sz[:2], rtol=1e-12), s
        assert np.all(y[2] == 0.0) and np.all(S[2] == 0.0)
