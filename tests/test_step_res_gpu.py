"""GPU parity of the residual walk (mk_q4k_step_res): the persistent step with
real-layer epilogues (RMSNorm with weights, residual adds, SiLU * up).

The fp32 residual stream is rebuilt on the host from h0 and the GPU's own
outputs (h_mid = h + o and h_out = h_mid + down, fp32 additions, so they must
match bit for bit). Every phase input must be the binary16 cast of its fp32
value (h * g, q, h_mid * g: bit for bit; silu(gate) * up: within one binary16
step, since the device exp may differ from numpy's in the last place). Every
matrix is checked against its own binary16 input by the oracle: the normed
ones (q, k, v, gate, up) with the row scale 1 / sqrt(mean(h^2) + 1e-6) of the
residual, the others plain, within |y - y_ref| <= 1e-4 * S."""
import numpy as np
import pytest

import oracle
from synth.stack import ResStack, shapes, MATRIX_ORDER

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)

import bit_weight_streaming_amd as mk  # noqa: E402

DEV = "cuda:0"
SMALL = shapes(H=512, Nq=768, Nkv=256, F=1280)
RAGGED = shapes(H=768, Nq=512, Nkv=200, F=1024)


def run_res(stack, reps=1):
    descs = stack.layer_descs()
    nbytes = mk.step_workspace_bytes(descs[0], stack.n_layers, stack.M)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    for _ in range(reps):
        mk.step_res(descs, stack.io, stack.norms, stack.h0, ws, stack.M)
    torch.cuda.synchronize()
    st = mk.step_status(ws)
    assert st == 0, f"device status {st}: {mk.strerror(st)}"
    return ws


def f16_bits(v32):
    return oracle.f64_to_f16(np.asarray(v32, dtype=np.float32).astype(np.float64))


def check_cast(x_gpu, v32, what, steps=0):
    """x_gpu (binary16) against the round-to-nearest-even cast of v32 (fp32):
    equal, or at most `steps` binary16 steps apart."""
    v32 = np.asarray(v32, dtype=np.float32)
    assert np.all(np.isfinite(v32)), what
    ref = f16_bits(v32).astype(np.int32)
    got = np.asarray(x_gpu).view(np.uint16).astype(np.int32)
    # binary16 bit patterns to a monotone integer line (sign-magnitude)
    def line(b):
        return np.where(b & 0x8000, -(b & 0x7FFF), b & 0x7FFF)
    d = np.abs(line(ref) - line(got))
    assert d.max() <= steps, f"{what}: {np.count_nonzero(d > steps)} of {d.size} values off"
    return int(np.count_nonzero(d))


def check_res_stack(stack, check_layers=None, ncols=None, seed=0):
    rng = np.random.default_rng(seed)
    check_layers = set(range(stack.n_layers) if check_layers is None else check_layers)
    h = stack.h0.cpu().numpy()
    worst = 0.0
    off = 0
    for l in range(stack.n_layers):
        io = stack.io[l]
        xs = [io["x"][p].cpu().numpy() for p in range(4)]
        ys = [io["y"][t].cpu().numpy() for t in range(7)]
        h_mid, h_out = (io["h"][j].cpu().numpy() for j in range(2))
        g_attn, g_ffn = (stack.norms[l][j].cpu().numpy() for j in range(2))
        for t in range(7):
            assert np.all(np.isfinite(ys[t])), (l, MATRIX_ORDER[t])
        # the residual stream: fp32 additions of the GPU's own outputs
        assert np.array_equal(h_mid, h + ys[3]), f"layer {l} h_mid"
        assert np.array_equal(h_out, h_mid + ys[6]), f"layer {l} h_out"
        # the phase inputs
        check_cast(xs[0], h * g_attn, f"layer {l} cast(h*g_attn)")
        check_cast(xs[1], ys[0], f"layer {l} cast(q)")
        check_cast(xs[2], h_mid * g_ffn, f"layer {l} cast(h_mid*g_ffn)")
        g, u = ys[4], ys[5]
        # exp(-g) may overflow to inf for very negative g: silu's factor is then 0
        with np.errstate(over="ignore"):
            silu_u = g / (np.float32(1) + np.exp(-g)) * u
        off += check_cast(xs[3], silu_u, f"layer {l} cast(silu(gate)*up)", steps=1)
        if l in check_layers:
            r_attn = oracle.rms_inv(h.astype(np.float64))
            r_ffn = oracle.rms_inv(h_mid.astype(np.float64))
            for t, name in enumerate(MATRIX_ORDER):
                N, K = stack.shp[name]
                if ncols is None or ncols >= N:
                    cols = np.arange(N)
                else:
                    cols = np.unique(np.concatenate([rng.choice(N, ncols, replace=False),
                                                     [0, N - 1]]))
                W = stack.host_rows(l, name, cols)
                if name in ("q", "k", "v"):
                    y_ref, S = oracle.gemm_rms(W, xs[0], r_attn)
                elif name == "o":
                    y_ref, S = oracle.gemm(W, xs[1])
                elif name in ("gate", "up"):
                    y_ref, S = oracle.gemm_rms(W, xs[2], r_ffn)
                else:
                    y_ref, S = oracle.gemm(W, xs[3])
                ok, w, nbad = oracle.within_bound(ys[t][:, cols].astype(np.float64), y_ref, S)
                assert ok, f"layer {l} {name}: {nbad} outside the bound, worst {w:.3e}"
                worst = max(worst, w)
        h = h_out
    return worst, off


@pytest.mark.parametrize("M", [12, 1, 16, 40])
def test_res_small_stack_all_columns(M):
    stack = ResStack(3, M, SMALL, seed=30 + M, device=DEV)
    run_res(stack)
    worst, off = check_res_stack(stack)
    print(f"M={M} worst |err|/S = {worst:.3e}, silu casts one step off: {off}")


def test_res_ragged_stack():
    stack = ResStack(2, 12, RAGGED, seed=41, device=DEV)
    run_res(stack)
    check_res_stack(stack)


def test_res_deterministic_and_repeatable():
    stack = ResStack(2, 12, SMALL, seed=42, device=DEV)
    run_res(stack)
    first = [[t.clone() for t in io["y"] + io["x"] + io["h"]] for io in stack.io]
    run_res(stack, reps=2)
    for a, io in zip(first, stack.io):
        for u, v in zip(a, io["y"] + io["x"] + io["h"]):
            assert torch.equal(u, v)


def test_res_rows_bit_identical_alone_or_stacked():
    stack = ResStack(2, 12, SMALL, seed=45, device=DEV)
    run_res(stack)
    for r in (0, 11):
        one = ResStack(2, 1, SMALL, seed=45, device=DEV)
        one.h0.copy_(stack.h0[r:r + 1])
        run_res(one)
        for l in range(2):
            for a, b in zip(one.io[l]["y"] + one.io[l]["x"] + one.io[l]["h"],
                            stack.io[l]["y"] + stack.io[l]["x"] + stack.io[l]["h"]):
                assert torch.equal(a[0], b[r]), (r, l)


def test_res_rows_of_a_later_row_group_bit_identical():
    """Rows 16.. of a 20-row residual walk (the second row group) against
    the same rows walked alone."""
    stack = ResStack(2, 20, SMALL, seed=46, device=DEV)
    run_res(stack)
    tail = ResStack(2, 4, SMALL, seed=46, device=DEV)
    tail.h0.copy_(stack.h0[16:])
    run_res(tail)
    for l in range(2):
        for a, b in zip(tail.io[l]["y"] + tail.io[l]["x"] + tail.io[l]["h"],
                        stack.io[l]["y"] + stack.io[l]["x"] + stack.io[l]["h"]):
            assert torch.equal(a, b[16:]), l


def test_res_rejects_missing_norm():
    stack = ResStack(1, 4, SMALL, seed=43, device=DEV)
    descs = stack.layer_descs()
    ws = torch.empty(mk.step_workspace_bytes(descs[0], 1, 4), dtype=torch.uint8, device=DEV)
    with pytest.raises(mk.MkError) as e:
        mk.step_res(descs, stack.io, [(stack.norms[0][0], None)], stack.h0, ws, 4)
    assert e.value.code == mk.MK_EINVAL


def test_res_full_size_layers_sampled_columns():
    """Eight layers of the full 27B-class shapes at M=12, the launch the step
    benchmark uses; 4096 sampled columns per matrix (all of k and v) in the
    first and last layers, every residual and cast in full."""
    stack = ResStack(8, 12, seed=44, device=DEV)
    run_res(stack, reps=2)
    worst, off = check_res_stack(stack, check_layers=(0, 7), ncols=4096, seed=4321)
    print(f"full-size residual walk worst |err|/S = {worst:.3e}, silu casts one step off: {off}")


class _WorkloadResStack(ResStack):
    """The residual walk on the benchmark's own weight generator (not centred:
    the Q4_K blocks of d * sc * q - dmin * m with d, dmin ~ |N(0,1)| 1e-3)."""
    centered = False


def test_res_workload_weights_one_layer():
    """The residual walk on the workload's (uncentred) Q4_K weights: every
    output, residual and cast of one layer against the oracle, as for the
    centred stacks."""
    stack = _WorkloadResStack(1, 12, SMALL, seed=47, device=DEV)
    run_res(stack)
    worst, off = check_res_stack(stack)
    print(f"workload weights, one layer: worst |err|/S = {worst:.3e}, silu casts one step off: {off}")


def test_res_workload_weights_leave_the_range_and_say_so():
    """A second layer of those weights drives the residual stream past what the
    row statistics hold (the uncentred weights add a bias every matrix): the
    walk reports MK_ERANGE in its status word rather than a wrong result."""
    stack = _WorkloadResStack(2, 12, SMALL, seed=47, device=DEV)
    descs = stack.layer_descs()
    ws = torch.empty(mk.step_workspace_bytes(descs[0], 2, 12), dtype=torch.uint8, device=DEV)
    mk.step_res(descs, stack.io, stack.norms, stack.h0, ws, 12)
    torch.cuda.synchronize()
    assert mk.step_status(ws) == mk.MK_ERANGE


@pytest.mark.parametrize("form", ["iterator", "reload_stats"])
def test_res_walk_forms_agree_bit_for_bit(form):
    """The residual walk in the other forms of the walk (the record iterator
    instead of record tables; the normed phases' input statistics reloaded
    at the end of every phase): every output, residual and cast the same,
    bit for bit."""
    a = ResStack(2, 12, SMALL, seed=48, device=DEV)
    b = ResStack(2, 12, SMALL, seed=48, device=DEV)
    run_res(a)
    try:
        mk.step_set_walk_form(
            dict(iterator=mk.MK_WALK_ITERATOR, reload_stats=mk.MK_WALK_RELOAD_STATS)[form])
        run_res(b)
    finally:
        mk.step_set_walk_form(mk.MK_WALK_AUTO)
    for la, lb in zip(a.io, b.io):
        for u, v in zip(la["y"] + la["x"] + la["h"], lb["y"] + lb["x"] + lb["h"]):
            assert torch.equal(u, v)
    check_res_stack(b)
