"""GPU parity of the persistent decode-step walk (mk_q4k_step).

For every layer and matrix the oracle multiplies the row-standardized form of
the GPU's own binary16 phase input (io.x) by the Q4_K weights of the checked
columns and compares with the GPU output within |y - y_ref| <= 1e-4 * sum|w t|
(t the standardized input); every phase input must be, bit for bit, the
binary16 cast of the GPU's fp32 output that feeds it. Checking each matrix
against its own input keeps rounding differences from compounding along the
4*L chained products."""
import numpy as np
import pytest

import oracle
import synth
from synth.stack import Stack, shapes, MATRIX_ORDER

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)

import bit_weight_streaming_amd as mk  # noqa: E402

DEV = "cuda:0"
PHASE_OF = {"q": 0, "k": 0, "v": 0, "o": 1, "gate": 2, "up": 2, "down": 3}


def run_step(stack, reps=1):
    descs = stack.layer_descs()
    nbytes = mk.step_workspace_bytes(descs[0], stack.n_layers, stack.M)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    for _ in range(reps):
        mk.step(descs, stack.io, stack.x0, stack.x_out, ws, stack.M)
    torch.cuda.synchronize()
    st = mk.step_status(ws)
    assert st == 0, f"device status {st}: {mk.strerror(st)}"
    return ws


def check_cast(x_gpu, v32, what):
    """x_gpu (binary16) must be the round-to-nearest-even cast of v32 (fp32)."""
    v32 = np.asarray(v32, dtype=np.float32)
    assert np.all(np.isfinite(v32)), what
    ref = oracle.f64_to_f16(v32.astype(np.float64))
    got = np.asarray(x_gpu).view(np.uint16)
    bad = ref != got
    assert not bad.any(), f"{what}: {bad.sum()} of {bad.size} values differ from the binary16 cast"


def check_stack(stack, layers=None, ncols=None, seed=0, skip=()):
    rng = np.random.default_rng(seed)
    layers = range(stack.n_layers) if layers is None else layers
    x0 = stack.x0.cpu().numpy()
    worst = 0.0
    for l in layers:
        io = stack.io[l]
        xs = [io["x"][p].cpu().numpy() for p in range(4)]
        ys = [io["y"][t].cpu().numpy() for t in range(7)]
        for t in range(7):
            assert np.all(np.isfinite(ys[t])), (l, MATRIX_ORDER[t])
        # phase inputs: binary16 casts of the fp32 outputs that feed them
        if l == 0:
            assert np.array_equal(xs[0].view(np.uint16), x0.view(np.uint16))
        else:
            check_cast(xs[0], stack.io[l - 1]["y"][6].cpu().numpy(), f"layer {l} input")
        check_cast(xs[1], ys[0], f"layer {l} cast(q)")
        check_cast(xs[2], ys[3], f"layer {l} cast(o)")
        check_cast(xs[3], ys[4] * ys[5], f"layer {l} cast(gate*up)")   # fp32 product
        # every matrix against its own (standardized) input
        for t, name in enumerate(MATRIX_ORDER):
            if name in skip:
                continue
            N, K = stack.shp[name]
            if ncols is None or ncols >= N:
                cols = np.arange(N)
            else:
                cols = np.unique(np.concatenate([rng.choice(N, ncols, replace=False), [0, N - 1]]))
            W = stack.host_rows(l, name, cols)
            ref = oracle.q6k_gemm_std if stack.is_q6(l, name) else oracle.gemm_std
            y_ref, S = ref(W, xs[PHASE_OF[name]])
            ok, w, nbad = oracle.within_bound(ys[t][:, cols].astype(np.float64), y_ref, S)
            assert ok, f"layer {l} {name}: {nbad} outside the bound, worst {w:.3e}"
            worst = max(worst, w)
    return worst


def check_out(stack):
    check_cast(stack.x_out.cpu().numpy(), stack.io[-1]["y"][6].cpu().numpy(), "x_out")


SMALL = shapes(H=512, Nq=768, Nkv=256, F=1280)
RAGGED = shapes(H=768, Nq=512, Nkv=200, F=1024)


@pytest.mark.parametrize("M", [12, 1, 5, 16, 32, 33, 64])
def test_small_stack_all_columns(M):
    stack = Stack(3, M, SMALL, seed=M, device=DEV)
    run_step(stack)
    worst = check_stack(stack)
    check_out(stack)
    print(f"M={M} worst |err|/S = {worst:.3e}")


def test_ragged_kv_stack():
    stack = Stack(2, 12, RAGGED, seed=7, device=DEV)
    run_step(stack)
    check_stack(stack)


def test_step_deterministic_and_repeatable():
    stack = Stack(2, 12, SMALL, seed=3, device=DEV)
    ws = run_step(stack)
    first = [[y.clone() for y in io["y"]] for io in stack.io]
    xo = stack.x_out.clone()
    descs = stack.layer_descs()
    for _ in range(3):
        mk.step(descs, stack.io, stack.x0, stack.x_out, ws, stack.M)
    torch.cuda.synchronize()
    assert mk.step_status(ws) == 0
    for l, io in enumerate(stack.io):
        for t in range(7):
            assert torch.equal(io["y"][t], first[l][t]), (l, t)
    assert torch.equal(stack.x_out, xo)


def test_step_rejects_bad_chain():
    stack = Stack(1, 4, SMALL, seed=1, device=DEV)
    descs = stack.layer_descs()
    bad = [dict(descs[0])]
    w, N, K, t = bad[0]["o"]
    bad[0]["o"] = (w, N, K + 256, t)        # o.K != q.N
    ws = torch.empty(1 << 20, dtype=torch.uint8, device=DEV)
    with pytest.raises(mk.MkError) as e:
        mk.step(bad, stack.io, stack.x0, stack.x_out, ws, 4)
    assert e.value.code == mk.MK_EINVAL
    with pytest.raises(mk.MkError) as e:
        mk.step(descs, stack.io, stack.x0, stack.x_out, ws[:16], 4)
    assert e.value.code == mk.MK_EWORKSPACE


def test_second_step_on_new_input_reads_fresh_values():
    """Two steps over the same buffers and workspace with different layer-0
    inputs: every value of the second must follow from its own input (a
    cached line left over from the first step would fail the checks)."""
    stack = Stack(3, 12, SMALL, seed=21, device=DEV)
    ws = run_step(stack)
    stack.x0.copy_(torch.from_numpy(synth.activations(99, 12, stack.H)).to(DEV))
    mk.step(stack.layer_descs(), stack.io, stack.x0, stack.x_out, ws, stack.M)
    torch.cuda.synchronize()
    assert mk.step_status(ws) == 0
    check_stack(stack)
    check_out(stack)


def test_rows_bit_identical_alone_or_stacked():
    """The K slices of every phase are chosen for 16 rows whatever M is, each
    row's statistics are exact integer sums of its own values, and nothing
    else mixes rows: a row walked alone gives every output and every cast of
    the 12-row walk bit for bit."""
    stack = Stack(2, 12, SMALL, seed=51, device=DEV)
    run_step(stack)
    for r in (0, 7, 11):
        one = Stack(2, 1, SMALL, seed=51, device=DEV)
        one.x0.copy_(stack.x0[r:r + 1])
        run_step(one)
        for l in range(2):
            for a, b in zip(one.io[l]["y"] + one.io[l]["x"], stack.io[l]["y"] + stack.io[l]["x"]):
                assert torch.equal(a[0], b[r]), (r, l)
        assert torch.equal(one.x_out[0], stack.x_out[r])


def test_decode_rows_stacked_with_a_prefill_chunk():
    """A mixed step: 12 decode rows (4 agents x 3) stacked with a 32-row
    prefill chunk of a new prompt, 44 rows in one call (three row groups:
    the decode rows share the first with 4 prefill rows). Every output and
    every cast of each part is, bit for bit, what the part gives walked alone
    (12 rows; 32 rows), and the stacked call matches the oracle."""
    dec = Stack(2, 12, SMALL, seed=61, device=DEV)
    pre = Stack(2, 32, SMALL, seed=61, device=DEV)
    pre.x0.copy_(torch.from_numpy(synth.activations(62, 32, dec.H)).to(DEV))
    both = Stack(2, 44, SMALL, seed=61, device=DEV)
    both.x0.copy_(torch.cat([dec.x0, pre.x0]))
    for s in (dec, pre, both):
        run_step(s)
    for l in range(2):
        for a, b, c in zip(dec.io[l]["y"] + dec.io[l]["x"], pre.io[l]["y"] + pre.io[l]["x"],
                           both.io[l]["y"] + both.io[l]["x"]):
            assert torch.equal(c[:12], a), l
            assert torch.equal(c[12:], b), l
    assert torch.equal(both.x_out[:12], dec.x_out)
    assert torch.equal(both.x_out[12:], pre.x_out)
    check_stack(both)
    check_out(both)


def test_full_size_layers_64_rows():
    """Two layers of the full 27B-class shapes at M = 64 (four row groups),
    1024 sampled columns per matrix (all of k and v), every cast in full."""
    stack = Stack(2, 64, seed=63, device=DEV)
    run_step(stack)
    worst = check_stack(stack, ncols=1024, seed=64)
    check_out(stack)
    print(f"full-size layers, M=64: worst |err|/S = {worst:.3e}")


def test_full_stack_sampled_columns():
    """The 64-layer stack at M=12 (12.27 GB of weights), as the benchmark runs
    it; every matrix checked on a seeded subset of 4096 columns (all columns
    of k and v) against its own binary16 input, every cast in full."""
    stack = Stack(64, 12, seed=0, device=DEV)
    run_step(stack, reps=2)
    worst = check_stack(stack, ncols=4096, seed=1234)
    check_out(stack)
    print(f"full stack worst |err|/S = {worst:.3e}")


class _CustomStack(Stack):
    """A Stack whose listed (layer, matrix) weights are replaced by given
    Q4_K rows (repacked into tile records like the generated ones)."""

    def __init__(self, overrides, *args, **kw):
        super().__init__(*args, **kw)
        self.overrides = overrides
        for (l, name), rows in overrides.items():
            N, K = self.shp[name]
            assert rows.shape == (N, K // 256 * 144)
            self.weights[l][name] = mk.repack(torch.from_numpy(np.ascontiguousarray(rows)).to(DEV),
                                              N, K)
        torch.cuda.synchronize()

    def host_rows(self, layer, name, rows):
        if (layer, name) in self.overrides:
            return self.overrides[(layer, name)][np.asarray(rows)]
        return super().host_rows(layer, name, rows)


def test_one_layer_min_term_edge_cases():
    """One layer whose input has 32-value sub-blocks summing past binary16's
    range (+-2100, 65504 would overflow the statistics' fixed point, so 6000)
    and whose q matrix starts with 16 columns of exactly cancelling weights
    (w = 0) and 16 of nearly cancelling ones. Every output is checked against
    the oracle: the cancelling columns within 1e-4 of the size of the factored
    terms (r * (sum (|d sc q| + |dmin m|) |x| + |mean * colsum|)), the rest
    within the usual bound."""
    M = 12
    shp = SMALL
    Nq, H = shp["q"]
    gen = synth.q4k_rows(synth.weight_key(31, 0, 0), H, 0, Nq)
    q_rows = gen.copy()
    q_rows[:16] = np.frombuffer(_cancel_block_bytes(0x4B80) * (H // 256), dtype=np.uint8).reshape(1, -1)
    q_rows[16:32] = np.frombuffer(_cancel_block_bytes(0x4B81) * (H // 256), dtype=np.uint8).reshape(1, -1)
    stack = _CustomStack({(0, "q"): q_rows}, 1, M, shp, seed=31, device=DEV)
    X = synth.activations(31, M, H).astype(np.float32)
    for m in range(M):
        for i, v in enumerate((2100.0, -2100.0, 6000.0)):
            j = (3 * m + 5 * i) % (H // 32)
            X[m, 32 * j:32 * j + 32] = v
    stack.x0 = torch.from_numpy(X.astype(np.float16)).to(DEV)
    run_step(stack)
    x_a = stack.io[0]["x"][0].cpu().numpy()
    yq = stack.io[0]["y"][0].cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(yq))
    y_ref, S = oracle.gemm_std(q_rows[:32], x_a)
    mean, r = oracle.row_moments(x_a)
    F = oracle.factored_size(q_rows[:32], x_a, mean=mean, r=r)
    ok, worst_f, nbad = oracle.within_bound(yq[:, :32], y_ref, F)
    assert ok, f"cancelling columns: {nbad} outside 1e-4 * F, worst {worst_f:.3e}"
    # every other column and matrix against the usual bound
    rest = np.arange(32, Nq)
    y_ref, S = oracle.gemm_std(q_rows[rest], x_a)
    ok, worst, nbad = oracle.within_bound(yq[:, rest], y_ref, S)
    assert ok, f"q columns 32..: {nbad} outside the bound, worst {worst:.3e}"
    stack_checked = check_stack(stack, skip=("q",))
    print(f"one layer, edge cases: cancelling worst |err|/F {worst_f:.3e}, "
          f"others {max(worst, stack_checked):.3e}")


def _cancel_block_bytes(dmin_bits):
    """d = 1, every scale and min 63, every quant 15 (see the GEMM tests)."""
    b = bytearray(144)
    b[0:2] = (0x3C00).to_bytes(2, "little")
    b[2:4] = int(dmin_bits).to_bytes(2, "little")
    b[4:16] = bytes([0xFF] * 12)
    b[16:] = bytes([0xFF] * 128)
    return bytes(b)


# --- Q4_K_M layers: v and down in Q6_K in some layers ------------------------
def test_q6k_walk_records_layout():
    """The walk's Q6_K records hold, for lane l = c + 16 g of tile t and
    block b, the low nibbles of weights 64g + i / 64g + 32 + i (bytes 0..15)
    and 64g + 16 + i / 64g + 48 + i (bytes 1024..), the high bit pairs packed
    four to a byte, the scales of runs 4g..4g+3 and row c's d, with the
    column sums after the records (rebuilt here from the block definition)."""
    N, K = 37, 512
    W = synth.q6k_matrix(synth.key(81, 14, N, K), N, K)
    T = mk.q6k_step_repack(torch.from_numpy(W).to(DEV).reshape(-1), N, K).cpu().numpy()
    nt, KB = (N + 15) // 16, K // 256
    blocks = W.reshape(N, KB, 210)

    def low4(blk, k):
        h, j, l = k >> 7, (k & 127) >> 5, k & 31
        return (int(blk[64 * h + 32 * (j & 1) + l]) >> (4 * (j >> 1))) & 15

    def high2(blk, k):
        h, j, l = k >> 7, (k & 127) >> 5, k & 31
        return (int(blk[128 + 32 * h + l]) >> (2 * j)) & 3

    ref = np.zeros(nt * KB * 3360, dtype=np.uint8)
    for t in range(nt):
        for b in range(KB):
            rec = ref[(t * KB + b) * 3360:(t * KB + b + 1) * 3360]
            for lane in range(64):
                c, g = lane & 15, lane >> 4
                n = 16 * t + c
                if n >= N:
                    continue
                blk = blocks[n, b]
                k0 = 64 * g
                for i in range(16):
                    rec[16 * lane + i] = low4(blk, k0 + i) | (low4(blk, k0 + 32 + i) << 4)
                    rec[1024 + 16 * lane + i] = low4(blk, k0 + 16 + i) | (low4(blk, k0 + 48 + i) << 4)
                for m in range(4):
                    for bb in range(4):
                        rec[2048 + 16 * lane + 4 * m + bb] = (
                            high2(blk, k0 + 8 * m + bb) | (high2(blk, k0 + 32 + 8 * m + bb) << 2) |
                            (high2(blk, k0 + 8 * m + 4 + bb) << 4) | (high2(blk, k0 + 36 + 8 * m + bb) << 6))
                rec[3072 + 4 * lane:3072 + 4 * lane + 4] = blk[192 + 4 * g:192 + 4 * g + 4]
                rec[3328 + 2 * c:3330 + 2 * c] = blk[208:210]
    assert np.array_equal(T[:ref.size], ref)
    cs = T[ref.size:].view(np.float32)
    w = oracle.q6k_dequant_rows(W, K)
    want = np.zeros(nt * 16, dtype=np.float32)
    want[:N] = w.sum(axis=1).astype(np.float32)
    assert np.array_equal(cs, want)


Q6_MIXED = {(0, "v"), (1, "down"), (2, "v"), (2, "down")}


@pytest.mark.parametrize("M", [12, 1, 16])
def test_q6k_mixed_stack_all_columns(M):
    stack = Stack(3, M, SMALL, seed=71 + M, device=DEV, q6=Q6_MIXED)
    run_step(stack)
    worst = check_stack(stack)
    check_out(stack)
    print(f"mixed Q4_K/Q6_K, M={M}: worst |err|/S = {worst:.3e}")


def test_q6k_mixed_ragged_stack():
    """v with 200 columns (a ragged last tile) in Q6_K."""
    stack = Stack(2, 12, RAGGED, seed=74, device=DEV, q6={(0, "v"), (1, "v"), (1, "down")})
    run_step(stack)
    check_stack(stack)
    check_out(stack)


def test_q6k_mixed_rows_bit_identical_alone_or_stacked():
    stack = Stack(3, 12, SMALL, seed=75, device=DEV, q6=Q6_MIXED)
    run_step(stack)
    for r in (0, 11):
        one = Stack(3, 1, SMALL, seed=75, device=DEV, q6=Q6_MIXED)
        one.x0.copy_(stack.x0[r:r + 1])
        run_step(one)
        for l in range(3):
            for a, b in zip(one.io[l]["y"] + one.io[l]["x"], stack.io[l]["y"] + stack.io[l]["x"]):
                assert torch.equal(a[0], b[r]), (r, l)


def test_q6k_mixed_full_size_layers():
    """Three layers of the full 27B-class shapes at M = 12, with Q6_K v and
    down in a Q4_K_M-like pattern; 2048 sampled columns per matrix."""
    stack = Stack(3, 12, seed=76, device=DEV, q6={(0, "v"), (0, "down"), (2, "v"), (2, "down")})
    run_step(stack, reps=2)
    worst = check_stack(stack, ncols=2048, seed=77)
    check_out(stack)
    print(f"full-size mixed layers: worst |err|/S = {worst:.3e}")


def _outputs(stack):
    return [t.clone() for io in stack.io for t in io["y"] + io["x"]] + [stack.x_out.clone()]


WALK_FORMS = {
    "iterator": mk.MK_WALK_ITERATOR,
    "reload_stats": mk.MK_WALK_RELOAD_STATS,
    "iterator_reload_stats": mk.MK_WALK_ITERATOR | mk.MK_WALK_RELOAD_STATS,
}


@pytest.mark.parametrize("form", list(WALK_FORMS))
@pytest.mark.parametrize("case", ["small", "ragged", "q6k_mixed"])
def test_walk_forms_agree_bit_for_bit(case, form):
    """The forms of the walk compute the same products in the same order:
    the weight records read through per-wave record tables or the record
    iterator (kept for waves with more than 64 records), and the input
    statistics taken as staged or reloaded at the end of every phase (the
    path a phase takes when some workgroup's share was not yet in when it
    staged). Every output of the step must be the same, bit for bit, and the
    other form must pass the oracle check as well."""
    kw = dict(small=(SMALL, ()), ragged=(RAGGED, ()), q6k_mixed=(SMALL, Q6_MIXED))[case]
    shp, q6 = kw
    a = Stack(2, 12, shp, seed=90, device=DEV, q6=q6)
    b = Stack(2, 12, shp, seed=90, device=DEV, q6=q6)
    run_step(a)
    try:
        mk.step_set_walk_form(WALK_FORMS[form])
        run_step(b)
    finally:
        mk.step_set_walk_form(mk.MK_WALK_AUTO)
    for u, v in zip(_outputs(a), _outputs(b)):
        assert torch.equal(u, v)
    check_stack(b)


def test_walk_form_rejects_unknown_values():
    with pytest.raises(mk.MkError) as e:
        mk.step_set_walk_form(4)
    assert e.value.code == mk.MK_EINVAL
