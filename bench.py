#!/usr/bin/env python3
"""Benchmark of the Q4_K weight-streaming decode step on one MI355X.

One step is one launch of the persistent walk (mk_q4k_step) over the full
synthetic layer stack: 64 layers of q 5120->6144, k/v 5120->1024,
o 6144->5120, gate/up 5120->17408 and down 17408->5120 Q4_K matrices
(12,268,339,200 weight bytes), 12 stacked activation rows (four agents, each
one next token plus two draft tokens). Inputs are seeded and synthetic and
resident in HBM before timing starts.

Prints one JSON line: weight-stream GB/s (value), % of the 8 TB/s HBM peak,
row-tokens/s per decode step, a roofline object for the step kernel and the
CPU oracle timed on a bounded sample of the same workload.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--layers L] [--no-cpu]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0   # MI355X HBM3E peak, GB/s (decimal)
# HBM traffic of the step kernel as measured by rocprofv3 PMC runs; reported only
# while the kernel sources still hash to the value recorded there.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "q4k_step_m12_64layers_traffic.md")
KERNEL_SOURCES = ("q4k_step.hip", "q4k_step.h", "q4k_device.h")
COPY_BYTES = 1 << 30
METRIC = "weight-stream GB/s and % of HBM peak at M=12; rows*tokens/s per decode step"


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def algorithmic_bytes(stack) -> dict:
    """Bytes one step must move: every weight once, the layer input x0, and the
    per-layer outputs the step materialises (fp32 y of the seven matrices,
    binary16 phase inputs) plus x_out."""
    M, H = stack.M, stack.H
    shp = stack.shp
    w = stack.weight_bytes
    y = stack.n_layers * M * sum(N for N, _ in shp.values()) * 4
    x = stack.n_layers * M * (H + shp["q"][0] + H + shp["gate"][0]) * 2
    io = 2 * M * H * 2
    return {"weights": w, "y": y, "x": x, "io": io, "total": w + y + x + io}


def kernel_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "bit_weight_streaming_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(n_layers: int, M: int):
    """HBM bytes per launch from the committed counter summary, or None when it
    is absent, was taken on another workload or the kernel changed since."""
    try:
        with open(TRAFFIC_FILE) as fh:
            kv = dict(l.strip()[2:].split(" = ", 1) for l in fh if l.startswith("- ") and " = " in l)
    except OSError:
        return None
    if kv.get("kernel_source_sha256") != kernel_source_hash():
        return None
    if int(kv.get("n_layers", -1)) != n_layers or int(kv.get("M", -1)) != M:
        return None
    return int(kv["hbm_bytes_per_launch"])


def copy_calibration(steps: int) -> int:
    """Plain device-to-device copies of COPY_BYTES each (the reference kernel the
    PMC byte counters are scaled by)."""
    import torch
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": COPY_BYTES, "copy_bytes_written": COPY_BYTES,
                      "launches": steps}), flush=True)
    return 0


# Single-matrix GEMM configurations (mk_q4k_gemm on the plain row layout):
# (label, M, N, K). Each weight matrix is 50 MB, inside the 256 MB Infinity
# Cache, so timed launches rotate over GEMM_COPIES independent copies.
GEMM_CONFIGS = (
    ("tiny K=1024 N=256", 1, 256, 1024),
    ("gate/up K=5120 N=17408", 12, 17408, 5120),
    ("down K=17408 N=5120", 1, 5120, 17408),
    ("down K=17408 N=5120", 4, 5120, 17408),
    ("down K=17408 N=5120", 8, 5120, 17408),
    ("down K=17408 N=5120", 12, 5120, 17408),
    ("down K=17408 N=5120", 16, 5120, 17408),
    ("tiny K=1024 N=256", 64, 256, 1024),
    ("gate/up K=5120 N=17408", 64, 17408, 5120),
)
GEMM_COPIES = 12
FP16_MFMA_PEAK_TFLOPS = 2500.0


def gemm_bench(seed: int, reps: int = 60) -> list:
    """Time the single-matrix GEMM on each configuration, on the plain row
    layout (mk_q4k_gemm) and on the tile-record form (mk_q4k_gemm_tiled): HIP
    events around `reps` back-to-back launches cycling over GEMM_COPIES weight
    copies (>= 600 MB for the 50 MB matrices), after warm-up launches."""
    import torch
    import bit_weight_streaming_amd as mk
    import synth
    out = []
    cache = {}
    stream = torch.cuda.current_stream()

    def timed(fn, n):
        for i in range(n + 2):
            fn(i)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(reps):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e-3

    for label, M, N, K in GEMM_CONFIGS:
        if (N, K) not in cache:
            w = torch.from_numpy(synth.q4k_matrix(synth.key(seed, 7, N, K), N, K))
            copies = GEMM_COPIES if N * K >= 1 << 24 else 1
            rows = [w.to("cuda:0") for _ in range(copies)]
            cache[(N, K)] = (rows, [mk.repack(r, N, K) for r in rows])
        rows, tiles = cache[(N, K)]
        X = torch.from_numpy(synth.activations(seed, M, K)).to("cuda:0")
        Y = torch.empty((M, N), dtype=torch.float32, device="cuda:0")
        wbytes = N * (K // 256) * 144
        alg = wbytes + M * K * 2 + M * N * 4
        line = {"config": label, "M": M, "weight_copies": len(rows)}
        for name, fn in (("rows", lambda i: mk.gemm(rows[i % len(rows)], X, out=Y)),
                         ("tiles", lambda i: mk.gemm_tiled(tiles[i % len(tiles)], X, N, out=Y))):
            t = timed(fn, len(rows))
            gbs = wbytes / t / 1e9
            line[name] = {
                "us": round(t * 1e6, 2), "weight_GBps": round(gbs, 1),
                "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
                "roofline_frac": round(alg / t / 1e9 / HBM_PEAK_GBS, 4),
                "mfma_util": round(2.0 * M * N * K / t / 1e12 / FP16_MFMA_PEAK_TFLOPS, 4),
                "row_tokens_per_s": round(M / t, 1),
            }
            log(f"gemm {name:5s} {label} M={M}: {t * 1e6:.2f} us, {gbs:.1f} GB/s")
        out.append(line)
    return out


Q6K_CONFIGS = (("down K=17408 N=5120", 12, 5120, 17408), ("gate/up K=5120 N=17408", 12, 17408, 5120),
               ("down K=17408 N=5120", 64, 5120, 17408))
Q6K_COPIES = 6


def q6k_bench(seed: int, reps: int = 60) -> list:
    """Time the two Q6_K products at the layer shapes: mk_q6k_gemm_tiled on
    tile records (M <= 16 here) and mk_q6k_gemm_step, the persistent K-split
    product on the walk's records (its second launch, the slice reduction,
    included). HIP events around `reps` back-to-back calls cycling over
    Q6K_COPIES weight copies (about 440 MB, beyond the last-level cache).
    Algorithmic bytes: the Q6_K weights (210 B per 256) + X + Y."""
    import torch
    import bit_weight_streaming_amd as mk
    import synth
    dev = "cuda:0"
    stream = torch.cuda.current_stream()
    out = []
    for label, M, N, K in Q6K_CONFIGS:
        w = torch.from_numpy(synth.q6k_matrix(synth.key(seed, 14, N, K), N, K))
        X = torch.from_numpy(synth.activations(seed, M, K)).to(dev)
        Y = torch.empty((M, N), dtype=torch.float32, device=dev)
        wbytes = N * (K // 256) * 210
        alg = wbytes + M * K * 2 + M * N * 4
        forms = [("step records", lambda wd: mk.q6k_step_repack(wd, N, K), mk.q6k_gemm_step,
                  "q4k_gemm_kernel<%d, 2> + q4k_gemm_reduce" % ((M + 15) // 16))]
        if M <= 16:
            forms.insert(0, ("tile records", lambda wd: mk.q6k_repack(wd, N, K), mk.q6k_gemm_tiled,
                             "q6k_gemm_kernel<1, %d>" % (4 if ((N + 15) // 16 + 3) // 4 >= 256 else
                                                         2 if ((N + 15) // 16 + 1) // 2 >= 512 else 1)))
        for form, repack, gemm, kern in forms:
            recs = [repack(w.to(dev)) for _ in range(Q6K_COPIES)]
            for i in range(2 * Q6K_COPIES):
                gemm(recs[i % Q6K_COPIES], X, N, out=Y)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(stream)
            for i in range(reps):
                gemm(recs[i % Q6K_COPIES], X, N, out=Y)
            e1.record(stream)
            torch.cuda.synchronize()
            t = e0.elapsed_time(e1) / reps * 1e-3
            log(f"q6k {label} M={M} ({form}): {t * 1e6:.2f} us, {wbytes / t / 1e9:.1f} GB/s")
            out.append({"config": label, "M": M, "form": form, "us": round(t * 1e6, 2),
                        "weight_GBps": round(wbytes / t / 1e9, 1),
                        "roofline_frac": round(alg / t / 1e9 / HBM_PEAK_GBS, 4), "kernel": kern})
            del recs
    return out


ATTN_CONFIGS = (
    # (label, per-agent cache lengths, rows per agent); 48 query heads over 8
    # KV heads of 128 dims, a shared pool of 8,256 pages (132k tokens)
    ("4 agents x 3 rows, 9k/27k/41k/55k tokens (132k pool full)", (9000, 27000, 41000, 55000), 3),
    ("1 agent x 3 rows, 131k tokens", (131072,), 3),
    ("4 agents x 3 rows, 2k tokens each", (2048,) * 4, 3),
)
ATTN_POOL_PAGES = 8256
ATTN_POOL_COPIES = 3


def attn_bench(seed: int, reps: int = 30) -> list:
    """Time one layer's decode attention (mk_q8_attn_decode: the split kernel
    and the merge) over the 132k-token q8_0 pool, with HIP events around
    `reps` back-to-back calls cycling over ATTN_POOL_COPIES copies of the pool
    (861 MB, beyond the last-level cache). Algorithmic bytes per call: every
    page-head a call reads (4352 B each) plus Q, O and the block table."""
    import torch
    import bit_weight_streaming_amd as mk
    import synth
    dev = "cuda:0"
    H, KV = 48, 8
    pool_np = synth.q8_pool(seed, ATTN_POOL_PAGES, KV)
    pools = [torch.from_numpy(pool_np).to(dev) for _ in range(ATTN_POOL_COPIES)]
    del pool_np
    stream = torch.cuda.current_stream()
    out = []
    for label, lengths, rows in ATTN_CONFIGS:
        table, _, row_len = synth.attn_layout(seed, lengths, rows, ATTN_POOL_PAGES)
        M = len(lengths) * rows
        Q = torch.from_numpy(synth.f16_normal(synth.key(seed, 77, M, H), M * H * 128)
                             .reshape(M, H, 128)).to(dev)
        tb, rl = torch.from_numpy(table).to(dev), torch.from_numpy(row_len).to(dev)
        ws = torch.empty(mk.attn_workspace_bytes(table.shape[0], table.shape[1], KV),
                         dtype=torch.uint8, device=dev)
        O = torch.empty((M, H, 128), dtype=torch.float32, device=dev)

        def call(i):
            mk.attn_decode(Q, pools[i % len(pools)], tb, rl, rows, KV, workspace=ws, out=O)

        for i in range(2 * len(pools)):
            call(i)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(reps):
            call(i)
        e1.record(stream)
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) / reps * 1e-3
        pages = sum((n + 15) // 16 for n in lengths)
        kv_bytes = pages * KV * 4352
        alg = kv_bytes + M * H * 128 * (2 + 4) + table.size * 4 + M * 4
        gbs = alg / t / 1e9
        log(f"attn {label}: {t * 1e6:.2f} us, {gbs:.1f} GB/s")
        out.append({"config": label, "M": M, "heads": f"{H}/{KV}", "kv_bytes": kv_bytes,
                    "us": round(t * 1e6, 2), "GBps": round(gbs, 1),
                    "roofline_frac": round(gbs / HBM_PEAK_GBS, 4),
                    "kernels": "q8_attn_kernel + q8_attn_merge"})
    return out


TL_NAMES = ("A", "B", "C", "D")


def timeline(args) -> int:
    """Per-boundary breakdown of the walk from the timeline build of the
    library (libmkq4k_timeline.so: the same kernels storing the wall clock,
    100 MHz, at five points of every phase of every workgroup). For each phase
    boundary, times are relative to the last workgroup's compute end of the
    producing phase; medians over the layers (first and last skipped)."""
    import numpy as np
    import torch
    import bit_weight_streaming_amd as mk
    mk.LIB_PATH = mk.TIMELINE_LIB_PATH
    from synth.stack import Stack
    torch.cuda.set_device(0)
    cus = json.loads(mk.device_info())["cus"]
    stack = Stack(args.layers, args.M, seed=args.seed, device="cuda:0")
    descs = stack.layer_descs()
    ws = torch.empty(mk.step_workspace_bytes(descs[0], args.layers, args.M), dtype=torch.uint8,
                     device="cuda:0")
    off = mk.step_timeline_offset(descs[0], args.layers, args.M)
    if off < 0:
        log("the loaded library has no timeline stamps")
        return 1
    for _ in range(args.warmup + 1):
        mk.step(descs, stack.io, stack.x0, stack.x_out, ws, args.M)
    torch.cuda.synchronize()
    if mk.step_status(ws) != 0:
        log(f"device status {mk.step_status(ws)}")
        return 1
    L, G = args.layers, cus
    raw = ws[off:off + L * 4 * G * 64].cpu().numpy().view(np.int64).reshape(L, 4, G, 8)
    t = raw[..., :5].astype(np.float64) / 100.0   # microseconds
    START, COMPUTED, PUBLISHED, FINISHED, SEEN = range(5)
    rows = []
    layer_us = np.diff(t[:, 3, :, COMPUTED].max(axis=1))
    for p in range(4):
        ref = t[:, p, :, COMPUTED].max(axis=1)               # last compute end, per layer
        med_end = np.median(t[:, p, :, COMPUTED], axis=1)
        pub = t[:, p, :, PUBLISHED].max(axis=1) - ref
        fin = t[:, p, :, FINISHED].max(axis=1) - ref
        seen_med = np.median(t[:, p, :, SEEN], axis=1) - ref
        seen_max = t[:, p, :, SEEN].max(axis=1) - ref
        nxt = np.full(L, np.nan)
        nxt_max = np.full(L, np.nan)
        if p < 3:
            nxt = np.median(t[:, p + 1, :, START], axis=1) - ref
            nxt_max = t[:, p + 1, :, START].max(axis=1) - ref
        else:
            nxt[:-1] = np.median(t[1:, 0, :, START], axis=1) - ref[:-1]
            nxt_max[:-1] = t[1:, 0, :, START].max(axis=1) - ref[:-1]
        span = np.median(t[:, p, :, COMPUTED] - t[:, p, :, START], axis=1)
        sel = slice(1, L - 1)
        rows.append({
            "boundary": f"{TL_NAMES[p]} -> {TL_NAMES[(p + 1) % 4]}",
            "compute_span_median_us": round(float(np.median(span[sel])), 2),
            "compute_end_spread_us": round(float(np.median((ref - med_end)[sel])), 2),
            "last_partial_published_us": round(float(np.median(pub[sel])), 2),
            "last_tile_finished_us": round(float(np.median(fin[sel])), 2),
            "done_seen_median_us": round(float(np.median(seen_med[sel])), 2),
            "done_seen_last_us": round(float(np.median(seen_max[sel])), 2),
            "next_compute_start_median_us": round(float(np.nanmedian(nxt[sel])), 2),
            "next_compute_start_last_us": round(float(np.nanmedian(nxt_max[sel])), 2),
        })
    out = {"timeline": {"workload": f"{L} layers, M={args.M}", "workgroups": G,
                        "layer_us_median": round(float(np.median(layer_us[1:-1])), 2),
                        "boundaries": rows}}
    for r in rows:
        log(f"{r['boundary']}: span {r['compute_span_median_us']} us, end spread "
            f"{r['compute_end_spread_us']}, published {r['last_partial_published_us']}, finished "
            f"{r['last_tile_finished_us']}, done seen {r['done_seen_median_us']} (last "
            f"{r['done_seen_last_us']}), next start {r['next_compute_start_median_us']} (last "
            f"{r['next_compute_start_last_us']})")
    log(f"layer: {out['timeline']['layer_us_median']} us (median)")
    print(json.dumps(out), flush=True)
    return 0


CEILING_BYTES = 12 << 30
CEILING_GRIDS = (256, 512, 1024)


def hbm_ceiling(reps: int = 3) -> dict:
    """The read bandwidth the chip reaches: mk_hbm_read_probe (every byte of a
    12 GiB buffer read once with 16-byte nontemporal loads, one contiguous
    share per workgroup) timed with HIP events over `reps` back-to-back
    launches, for a few grid sizes; the best is the measured ceiling."""
    import torch
    import bit_weight_streaming_amd as mk
    buf = torch.empty(CEILING_BYTES, dtype=torch.uint8, device="cuda:0")
    out = torch.empty(max(CEILING_GRIDS), dtype=torch.int32, device="cuda:0")
    stream = torch.cuda.current_stream()
    best = None
    per_grid = {}
    for grid in CEILING_GRIDS:
        mk.hbm_read_probe(buf, out, grid)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            mk.hbm_read_probe(buf, out, grid)
        e1.record(stream)
        torch.cuda.synchronize()
        gbs = CEILING_BYTES * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
        per_grid[grid] = round(gbs, 1)
        log(f"read ceiling probe, grid {grid} x 512: {gbs:.1f} GB/s")
        if best is None or gbs > best[0]:
            best = (gbs, grid)
    del buf
    return {"GBps": round(best[0], 1), "grid": best[1], "bytes": CEILING_BYTES, "reps": reps,
            "per_grid": per_grid,
            "kernel": "hbm_read_kernel (16-byte nontemporal loads, contiguous share per workgroup)"}


def cpu_baseline(stack, budget_s: float = 20.0) -> dict:
    """Time the fp64 oracle (as it stands) on the same decode step: layers
    chained through binary16 casts as the GPU walks them, each matrix applied
    to its row-standardized input, every column of every matrix, as many
    leading layers as fit in about budget_s of oracle time. Generating the
    weights on the host is input plumbing and is not timed."""
    import numpy as np
    import oracle
    import synth
    from synth.stack import MATRIX_ORDER
    M, shp = stack.M, stack.shp

    def cast(v):
        return oracle.f64_to_f16(v).view(np.float16)

    def rows(l, name):
        N, K = shp[name]
        return synth.q4k_rows(synth.weight_key(stack.seed, l, MATRIX_ORDER.index(name)), K, 0, N)

    x = synth.activations(stack.seed, M, stack.H)
    elapsed, done_bytes, layers = 0.0, 0, 0
    while layers < stack.n_layers:
        W = {n: rows(layers, n) for n in MATRIX_ORDER}
        t0 = time.perf_counter()
        yq = oracle.gemm_std(W["q"], x)[0]
        oracle.gemm_std(W["k"], x)
        oracle.gemm_std(W["v"], x)
        yo = oracle.gemm_std(W["o"], cast(yq))[0]
        xc = cast(yo)
        gu = oracle.gemm_std(W["gate"], xc)[0] * oracle.gemm_std(W["up"], xc)[0]
        x = cast(oracle.gemm_std(W["down"], cast(gu))[0])
        dt = time.perf_counter() - t0
        elapsed += dt
        done_bytes += sum(w.nbytes for w in W.values())
        layers += 1
        if elapsed + dt > budget_s:
            break
    gbs = done_bytes / elapsed / 1e9
    return {
        "value": round(gbs, 4),
        "unit": "GB/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": (f"the first {layers} of {stack.n_layers} layers of the same step, chained through "
                   f"binary16 casts, all columns of all 7 matrices, M={M}: {done_bytes / 1e9:.3f} GB of Q4_K "
                   f"weights in {elapsed:.2f} s (fp64 dequantize + naive matmul, OpenMP over "
                   f"columns); row-tokens/s at this rate "
                   f"{M * gbs * 1e9 / stack.weight_bytes:.4f}"),
    }


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--layers", type=int, default=64)
    ap.add_argument("--M", type=int, default=12)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-gemm", action="store_true", help="skip the single-matrix GEMM lines")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run plain 1 GiB copies (scale for the PMC byte counters)")
    ap.add_argument("--gemm-only", action="store_true",
                    help="only the single-matrix GEMM lines (no 64-layer stack)")
    ap.add_argument("--no-attn", action="store_true", help="skip the decode-attention lines")
    ap.add_argument("--ceiling", action="store_true",
                    help="only run the HBM read-ceiling probe (12 GiB, nontemporal 16-byte reads)")
    ap.add_argument("--no-ceiling", action="store_true", help="skip the read-ceiling probe")
    ap.add_argument("--timeline", action="store_true",
                    help="per-boundary time breakdown of the walk from the timeline build "
                         "(libmkq4k_timeline.so)")
    ap.add_argument("--q6k-only", action="store_true", help="only time the Q6_K product")
    ap.add_argument("--attn-only", action="store_true",
                    help="only time decode attention over the 132k-token q8_0 pool")
    ap.add_argument("--walk", choices=("std", "res"), default="std",
                    help="std: the standardized walk (the benchmark); res: the residual walk "
                         "(RMSNorm, residual adds, SiLU*up) on centred weights, timed alone")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the decode step is data parallel over agents, each GPU "
              "holding a full replica of the weights with nothing exchanged on the hot path; "
              "run it with --gpus 1 (multi-GPU runs are not part of this build).",
              file=sys.stderr)
        return 2

    if args.copy_calibration:
        return copy_calibration(args.steps)
    if args.timeline:
        return timeline(args)

    import torch
    import bit_weight_streaming_amd as mk
    from synth.stack import ResStack, Stack

    if args.gemm_only:
        torch.cuda.set_device(0)
        print(json.dumps({"gemm": gemm_bench(args.seed)}), flush=True)
        return 0
    if args.q6k_only:
        torch.cuda.set_device(0)
        print(json.dumps({"q6k": q6k_bench(args.seed)}), flush=True)
        return 0
    if args.attn_only:
        torch.cuda.set_device(0)
        print(json.dumps({"attn": attn_bench(args.seed)}), flush=True)
        return 0
    if args.ceiling:
        torch.cuda.set_device(0)
        print(json.dumps({"hbm_ceiling": hbm_ceiling()}), flush=True)
        return 0

    dev = "cuda:0"
    torch.cuda.set_device(0)
    log(f"device: {mk.device_info()}")
    t0 = time.time()
    res = args.walk == "res"
    stack = (ResStack if res else Stack)(args.layers, args.M, seed=args.seed, device=dev)
    torch.cuda.synchronize()
    log(f"stack ready: {args.layers} layers, {stack.weight_bytes / 1e9:.3f} GB of Q4_K weights "
        f"in {time.time() - t0:.1f} s")
    descs = stack.layer_descs()
    ws = torch.empty(mk.step_workspace_bytes(descs[0], args.layers, args.M), dtype=torch.uint8,
                     device=dev)

    def step():
        if res:
            mk.step_res(descs, stack.io, stack.norms, stack.h0, ws, args.M)
        else:
            mk.step(descs, stack.io, stack.x0, stack.x_out, ws, args.M)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    st = mk.step_status(ws)
    if st != 0:
        log(f"device status {st}: {mk.strerror(st)}")
        return 1
    log("warmup done")

    # the library launches on the stream it is given: the current torch stream,
    # so the events below are recorded on the launch stream itself
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    for a, b in ev:
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    st = mk.step_status(ws)
    if st != 0:
        log(f"device status {st}: {mk.strerror(st)}")
        return 1
    per_launch = [a.elapsed_time(b) for a, b in ev]
    ms = ev[0][0].elapsed_time(ev[-1][1]) / args.steps      # whole timed region
    t_launch = sum(per_launch) / len(per_launch) * 1e-3        # average launch duration
    t = ms * 1e-3
    ab = algorithmic_bytes(stack)
    gbs = stack.weight_bytes / t / 1e9
    log(f"{args.steps} steps: {ms:.3f} ms/step (events), launch avg {t_launch * 1e3:.3f} ms "
        f"(min {min(per_launch):.3f}, max {max(per_launch):.3f}), wall {wall / args.steps * 1e3:.3f} "
        f"ms/step, {gbs:.1f} GB/s weights")

    gemm = None
    if res:
        # the residual walk is timed alone: no GEMM lines, no CPU leg, no
        # committed counter record for it
        args.no_gemm = args.no_cpu = args.no_attn = True
    if not args.no_gemm:
        gemm = gemm_bench(args.seed)
    attn = q6k = None
    if not args.no_attn:
        attn = attn_bench(args.seed)
    if not args.no_gemm:
        q6k = q6k_bench(args.seed)

    ceiling = None
    if not res and not args.no_ceiling:
        ceiling = hbm_ceiling()

    cpu = None
    if not args.no_cpu:
        log("timing the CPU oracle on a bounded sample")
        cpu = cpu_baseline(stack)

    if res:
        # fp32 residual: h read and written twice per layer, h0, norm weights
        H = stack.H
        ab["total"] += args.layers * (4 * args.M * H * 4 + 2 * H * 4) + args.M * H * 4
    achieved = ab["total"] / t_launch / 1e9
    traffic = None if res else measured_traffic(args.layers, args.M)
    out = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "q4k*f16->f32",
        "data": "synthetic (seeded SplitMix64 Q4_K blocks, N(0,1) fp16 rows)",
        "config": {
            "workload": (f"decode step: {args.layers} layers x Q4_K q/k/v/o/gate/up/down "
                         f"(H=5120, q=6144, kv=1024, ffn=17408), M={args.M} stacked rows, "
                         f"one persistent launch"
                         + (", residual walk (RMSNorm, residual adds, SiLU*up; centred weights)"
                            if res else "")),
            "n_layers": args.layers,
            "M": args.M,
            "weight_bytes": stack.weight_bytes,
            "parallelism": "1 GPU",
        },
        "pct_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "hbm_ceiling": ceiling,
        "pct_of_measured_ceiling": round(100.0 * gbs / ceiling["GBps"], 2) if ceiling else None,
        "row_tokens_per_s": round(args.M / t, 1),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": ab["total"],
            "launch_ms": round(t_launch * 1e3, 4),
            "kernel": ("q4k_step_kernel<1>" if res else "q4k_step_kernel<0>")
                      + " (one launch = one decode step, all layers)",
        },
        "cpu_baseline": cpu,
        "gemm": gemm,
        "attn": attn,
        "q6k": q6k,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
