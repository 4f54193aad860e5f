"""GPU parity of decode attention over the paged q8_0 KV pool
(mk_q8_attn_decode) against the fp64 oracle: |O - O_ref| <= 1e-4 * S per
output element, S[d] = sum_i p_i |v_i[d]| + 2^-80 * (largest V scale the row
attends to: a floor at the edge of fp32's range), plus determinism and the
property that a row's result does not depend on the other rows in the call."""
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


def setup(seed, lengths, rows, n_heads, n_kv, n_pages):
    pool = synth.q8_pool(seed, n_pages, n_kv)
    table, _, row_len = synth.attn_layout(seed, lengths, rows, n_pages)
    M = len(lengths) * rows
    Q = synth.f16_normal(synth.key(seed, 77, M, n_heads), M * n_heads * 128).reshape(M, n_heads, 128)
    return pool, table, row_len, Q


def run(pool, table, row_len, Q, rows, n_kv):
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    O = mk.attn_decode(d(Q), d(pool), d(table), d(row_len), rows, n_kv)
    torch.cuda.synchronize()
    return O.cpu().numpy()


def check(pool, table, row_len, Q, rows, n_kv, O=None):
    if O is None:
        O = run(pool, table, row_len, Q, rows, n_kv)
    ra = np.repeat(np.arange(table.shape[0], dtype=np.int32), rows)
    O_ref, S = oracle.attn_decode(Q, pool, table, ra, row_len, n_kv)
    ok, worst, nbad = oracle.within_bound(O.astype(np.float64).reshape(len(Q), -1),
                                          O_ref.reshape(len(Q), -1), S.reshape(len(Q), -1))
    assert ok, f"{nbad} outside the bound, worst |err|/S = {worst:.3e}"
    return O, worst


@pytest.mark.parametrize("lengths,rows,H,KV", [
    ([70, 33, 150], 3, 4, 2),        # ragged pages, causal draft rows, 2 heads per KV head
    ([1, 16, 17, 1000], 1, 2, 2),    # single-token rows, page edges, one row per agent
    ([2100, 5], 2, 16, 1),           # 32 query vectors per KV head, several page groups
])
def test_small_configs_all_outputs(lengths, rows, H, KV):
    n_pages = sum((n + 15) // 16 for n in lengths) + 3
    pool, table, row_len, Q = setup(60 + H, lengths, rows, H, KV, n_pages)
    _, worst = check(pool, table, row_len, Q, rows, KV)
    print(f"lengths {lengths} rows {rows} heads {H}/{KV}: worst |err|/S = {worst:.3e}")


def test_four_agents_shared_132k_pool():
    """The decode step of the pages' setting: 4 agents x 3 rows, 48 query
    heads over 8 KV heads, caches of 9k-55k tokens in a shared pool of
    132k tokens (8,256 pages), every output against the oracle."""
    lengths = [9000, 27000, 41000, 55000]
    n_pages = 8256
    pool, table, row_len, Q = setup(61, lengths, 3, 48, 8, n_pages)
    O, worst = check(pool, table, row_len, Q, 3, 8)
    print(f"132k-token pool: worst |err|/S = {worst:.3e}")


def test_deterministic_and_rows_independent():
    """Repeated calls give the same bits; an agent's rows computed alone (a
    one-agent call with its page list) give the same bits as in the stack."""
    lengths = [300, 1200, 45]
    n_pages = 110
    pool, table, row_len, Q = setup(62, lengths, 3, 8, 2, n_pages)
    a = run(pool, table, row_len, Q, 3, 2)
    b = run(pool, table, row_len, Q, 3, 2)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    for ag in range(3):
        rows = slice(3 * ag, 3 * ag + 3)
        one = run(pool, table[ag:ag + 1], row_len[rows], Q[rows], 3, 2)
        assert np.array_equal(one.view(np.uint32), a[rows].view(np.uint32)), ag


def test_large_scales_and_peaked_scores():
    """V scales up to 8 and K scales that make the softmax nearly one-hot:
    the per-page power-of-two factor keeps the weights in binary16 range."""
    lengths = [500, 77]
    n_pages = 40
    pool, table, row_len, Q = setup(63, lengths, 3, 4, 2, n_pages)
    # scales: 64-byte groups of four tokens at 4096, K scales then V scales
    kat = np.concatenate([np.arange(4096 + 64 * g, 4096 + 64 * g + 32) for g in range(4)])
    vat = kat + 32
    def scaled(at, f):
        return (np.ascontiguousarray(pool[:, :, at]).view(np.float16) * np.float16(f)).view(np.uint8)
    pool[:, :, kat] = scaled(kat, 40.0)
    pool[:, :, vat] = scaled(vat, 64.0)
    assert np.all(np.isfinite(np.ascontiguousarray(pool[:, :, vat]).view(np.float16)))
    _, worst = check(pool, table, row_len, Q, 3, 2)
    print(f"large scales, peaked scores: worst per-element |err|/S = {worst:.3e}")


def _kscale_at(t, b):
    return 4096 + 64 * (t // 4) + 2 * (4 * (t % 4) + b)


def test_dominant_tokens_with_zero_values():
    """Three dominant tokens per agent whose scores stand about 11, 23 and 46
    nats above the rest, with value quants of 0 in the first 32 or 64 dims:
    those output dims are made of weights between about 2^-16 and 2^-70 of
    the largest one, which the value product must carry (its bfloat16 parts keep fp32's range) to
    meet the per-element bound."""
    lengths, rows, H, KV = [300, 200], 3, 4, 2
    n_pages = 40
    pool, table, row_len, Q = setup(65, lengths, rows, H, KV, n_pages)
    Q = np.abs(Q.astype(np.float32)).astype(np.float16)      # every query dim >= 0
    for a in range(len(lengths)):
        for t, ksc, zero_dims in ((5, 0.01, 32), (6, 0.02, 32), (7, 0.04, 64)):
            page, slot = table[a, t // 16], t % 16
            for h in range(KV):
                ph = pool[page, h]
                # K: quant +127 in every dim, one scale for the four blocks
                for d in range(128):
                    ph[1024 * ((d // 32) // 2) + 16 * (16 * ((d % 32) // 8) + slot)
                       + 8 * ((d // 32) % 2) + d % 8] = 127
                for b in range(4):
                    ph[_kscale_at(slot, b):_kscale_at(slot, b) + 2] = \
                        np.array([ksc], dtype=np.float16).view(np.uint8)
                # V: quant 0 in the first zero_dims dims
                for d in range(zero_dims):
                    ph[1024 * (2 + d // 64) + 16 * (16 * (slot // 4) + d % 16)
                       + 4 * ((d // 16) % 4) + slot % 4] = 0
    _, worst = check(pool, table, row_len, Q, rows, KV)
    print(f"dominant tokens with zero values: worst per-element |err|/S = {worst:.3e}")


def test_empty_cache_rows_are_zero():
    """An agent whose rows attend to no token (length 0, or a negative
    length, read as 0) gets exact zeros; the other agents' rows are
    unaffected and match the oracle."""
    lengths, rows, H, KV = [40, 300, 1], 3, 4, 2
    n_pages = 30
    pool, table, row_len, Q = setup(64, lengths, rows, H, KV, n_pages)
    row_len = row_len.copy()
    row_len[0:3] = [0, -5, 0]          # agent 0: nothing to attend to
    O, worst = check(pool, table, row_len, Q, rows, KV)
    assert np.all(O[0:3] == 0.0)
    print(f"empty-cache rows: worst |err|/S elsewhere = {worst:.3e}")
