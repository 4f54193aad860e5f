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


def cpu_baseline(stack, budget_s: float = 20.0) -> dict:
    """Time the fp64 oracle (as it stands) on layer 0 of the same workload:
    all seven matrices, all M rows, a prefix of each matrix's columns sized so
    the run stays near budget_s."""
    import numpy as np
    import oracle
    import synth
    from synth.stack import MATRIX_ORDER
    M = stack.M
    x = synth.activations(stack.seed, M, stack.H)
    # probe the rate on a small slice, then size the sample
    W = stack.host_rows(0, "q", np.arange(64))
    t0 = time.perf_counter()
    oracle.gemm(W, x)
    probe = max(time.perf_counter() - t0, 1e-4)
    weights_per_s = 64 * stack.shp["q"][1] / probe
    layer_weights = sum(N * K for N, K in stack.shp.values())
    frac = min(1.0, budget_s * weights_per_s / layer_weights)
    xs = {"q": x, "k": x, "v": x, "o": None, "gate": x, "up": x, "down": None}
    total_bytes = 0
    elapsed = 0.0
    for name in MATRIX_ORDER:
        N, K = stack.shp[name]
        n = max(16, int(N * frac))
        W = stack.host_rows(0, name, np.arange(n))
        xin = xs[name] if xs[name] is not None else synth.activations(stack.seed + 1, M, K)
        t0 = time.perf_counter()
        oracle.gemm(W, xin)
        elapsed += time.perf_counter() - t0
        total_bytes += W.nbytes
    gbs = total_bytes / elapsed / 1e9
    return {
        "value": round(gbs, 4),
        "unit": "GB/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": (f"layer 0, all 7 matrices, first {frac * 100:.1f}% of each matrix's columns, "
                   f"M={M}: {total_bytes / 1e6:.1f} MB of Q4_K weights in {elapsed:.2f} s "
                   f"(fp64 dequantize + naive matmul); row-tokens/s at this rate "
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
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the decode step is data parallel over agents, each GPU "
              "holding a full replica of the weights with nothing exchanged on the hot path; "
              "run it with --gpus 1 (multi-GPU runs are not part of this build).",
              file=sys.stderr)
        return 2

    import torch
    import bit_weight_streaming_amd as mk
    from synth.stack import Stack

    dev = "cuda:0"
    torch.cuda.set_device(0)
    log(f"device: {mk.device_info()}")
    t0 = time.time()
    stack = Stack(args.layers, args.M, seed=args.seed, device=dev)
    torch.cuda.synchronize()
    log(f"stack ready: {args.layers} layers, {stack.weight_bytes / 1e9:.3f} GB of Q4_K weights "
        f"in {time.time() - t0:.1f} s")
    descs = stack.layer_descs()
    ws = torch.empty(mk.step_workspace_bytes(descs[0], args.layers, args.M), dtype=torch.uint8,
                     device=dev)

    def step():
        mk.step(descs, stack.io, stack.x0, stack.x_out, ws, args.M)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    st = mk.step_status(ws)
    if st != 0:
        log(f"device status {st}: {mk.strerror(st)}")
        return 1
    log("warmup done")

    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    st = mk.step_status(ws)
    if st != 0:
        log(f"device status {st}: {mk.strerror(st)}")
        return 1
    ms = e0.elapsed_time(e1) / args.steps
    t = ms * 1e-3
    ab = algorithmic_bytes(stack)
    gbs = stack.weight_bytes / t / 1e9
    log(f"{args.steps} steps: {ms:.3f} ms/step (events), wall {wall / args.steps * 1e3:.3f} ms/step, "
        f"{gbs:.1f} GB/s weights")

    cpu = None
    if not args.no_cpu:
        log("timing the CPU oracle on a bounded sample")
        cpu = cpu_baseline(stack)

    achieved = ab["total"] / t / 1e9
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
                         f"one persistent launch"),
            "n_layers": args.layers,
            "M": args.M,
            "weight_bytes": stack.weight_bytes,
            "parallelism": "1 GPU",
        },
        "pct_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "row_tokens_per_s": round(args.M / t, 1),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": None,
            "algorithmic_bytes_per_launch": ab["total"],
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
