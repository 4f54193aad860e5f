"""Device-resident synthetic layer stacks for the decode-step walk.

Input plumbing only (no arithmetic of the method): weights come from the
seeded generator in ``synth.c`` (one stream per (seed, layer, matrix)), are
written into pinned host buffers and copied to the GPU; output buffers are
allocated empty. The real 27B-class shapes are hidden 5120, q 6144, k/v 1024,
FFN 17408 over 64 layers; smaller shapes serve the full-oracle tests.
"""
from __future__ import annotations

import numpy as np

from . import (LAYER_MATRICES, QK, BLOCK_BYTES, TAG_H0, TAG_NORM, activations, f32_normal, key,
               q4k_fill_ptr, q4k_fill_ptr_centered, q6k_rows, weight_key)

Q6K_BLOCK_BYTES = 210
TAG_Q6 = 14  # Q6_K matrices of a stack: (seed, TAG_Q6, layer, matrix index)

MATRIX_ORDER = ("q", "k", "v", "o", "gate", "up", "down")


def shapes(H=5120, Nq=6144, Nkv=1024, F=17408):
    """(name -> (N, K)) for one layer."""
    return {"q": (Nq, H), "k": (Nkv, H), "v": (Nkv, H), "o": (H, Nq),
            "gate": (F, H), "up": (F, H), "down": (H, F)}


MODEL_SHAPES = shapes()
assert all(MODEL_SHAPES[n] == (N, K) for n, K, N in LAYER_MATRICES)


def weight_bytes(shp, n_layers):
    return n_layers * sum(N * (K // QK) * BLOCK_BYTES for N, K in shp.values())


class Stack:
    """n_layers of Q4_K matrices plus the per-layer output buffers on `device`.

    The weights are kept on the device in the tile-record form the step walk
    reads (made by the library's repack call from the generated rows); the
    rows themselves can be regenerated on the host with host_rows(). `q6`
    lists (layer, name) matrices (name v or down, as in a Q4_K_M file) that
    are Q6_K instead, kept in the walk's Q6_K record form."""

    centered = False  # weight generator: the workload's, or centred (ResStack)

    def __init__(self, n_layers, M, shp=None, seed=0, device="cuda:0", q6=()):
        import torch
        self.torch = torch
        self.q6 = set(q6)
        assert all(name in ("v", "down") for _, name in self.q6)
        self.n_layers = n_layers
        self.M = M
        self.shp = dict(shp or MODEL_SHAPES)
        self.seed = seed
        self.device = device
        self.H = self.shp["q"][1]
        import bit_weight_streaming_amd as mk
        self.weights = []     # per layer: name -> uint8 tile-record tensor
        biggest = max(N * (K // QK) * BLOCK_BYTES for N, K in self.shp.values())
        pinned = torch.empty(biggest, dtype=torch.uint8, pin_memory=True)
        rows = torch.empty(biggest, dtype=torch.uint8, device=device)
        for l in range(n_layers):
            lay = {}
            for mi, name in enumerate(MATRIX_ORDER):
                N, K = self.shp[name]
                if (l, name) in self.q6:
                    r6 = torch.from_numpy(self.host_rows(l, name, np.arange(N))).to(device)
                    lay[name] = mk.q6k_step_repack(r6.reshape(-1), N, K)
                    torch.cuda.synchronize()
                    continue
                nbytes = N * (K // QK) * BLOCK_BYTES
                fill = q4k_fill_ptr_centered if self.centered else q4k_fill_ptr
                fill(weight_key(seed, l, mi), K, 0, N, pinned.data_ptr())
                rows[:nbytes].copy_(pinned[:nbytes], non_blocking=False)
                lay[name] = mk.repack(rows[:nbytes], N, K)
                torch.cuda.synchronize()
            self.weights.append(lay)
        del pinned, rows
        self.x0 = torch.from_numpy(activations(seed, M, self.H)).to(device)
        self.x_out = torch.empty((M, self.H), dtype=torch.float16, device=device)
        self.io = []
        F = self.shp["gate"][0]
        Nq = self.shp["q"][0]
        for l in range(n_layers):
            ys = [torch.empty((M, self.shp[n][0]), dtype=torch.float32, device=device)
                  for n in MATRIX_ORDER]
            xs = [torch.empty((M, w), dtype=torch.float16, device=device)
                  for w in (self.H, Nq, self.H, F)]
            self.io.append({"y": ys, "x": xs})

    def layer_descs(self):
        import bit_weight_streaming_amd as mk
        return [{n: (lay[n], self.shp[n][0], self.shp[n][1],
                     mk.MK_QTYPE_Q6_K if (l, n) in self.q6 else mk.MK_QTYPE_Q4_K)
                 for n in MATRIX_ORDER}
                for l, lay in enumerate(self.weights)]

    def is_q6(self, layer, name):
        return (layer, name) in self.q6

    def host_rows(self, layer, name, rows):
        """The bytes of the given weight rows of one matrix (regenerated): Q4_K,
        or Q6_K for the matrices listed in q6."""
        from . import q4k_rows, q4k_rows_centered
        N, K = self.shp[name]
        mi = MATRIX_ORDER.index(name)
        if (layer, name) in self.q6:
            full = q6k_rows(key(self.seed, TAG_Q6, layer, mi), K, 0, N)
            return full[np.asarray(rows)]
        gen = q4k_rows_centered if self.centered else q4k_rows
        full = gen(weight_key(self.seed, layer, mi), K, 0, N)
        return full[np.asarray(rows)]

    @property
    def weight_bytes(self):
        q6_extra = sum(self.shp[n][0] * (self.shp[n][1] // QK) * (Q6K_BLOCK_BYTES - BLOCK_BYTES)
                       for _, n in self.q6)
        return weight_bytes(self.shp, self.n_layers) + q6_extra


def norm_weights(seed, layer, which, H):
    """fp32 RMSNorm weight [H] of one layer (which: 0 before q/k/v, 1 before
    gate/up): 1 + 0.25 z, z ~ N(0,1)."""
    return (1.0 + 0.25 * f32_normal(key(seed, TAG_NORM, layer, which), H).astype(np.float64)
            ).astype(np.float32)


def residual_input(seed, M, H):
    """fp32 [M, H] residual stream entering layer 0: N(0,1) values."""
    return f32_normal(key(seed, TAG_H0, M, H), M * H).reshape(M, H)


class ResStack(Stack):
    """A Stack for the residual walk: centred weights (about zero mean, so
    the stream stays in range without a mean-removing norm), per-layer fp32
    RMSNorm weights, the fp32 residual input h0, and per-layer fp32 residual
    outputs h_mid (after o) and h_out (after down) next to the usual ones."""

    centered = True

    def __init__(self, n_layers, M, shp=None, seed=0, device="cuda:0"):
        super().__init__(n_layers, M, shp, seed, device)
        torch = self.torch
        H = self.H
        self.norms = [[torch.from_numpy(norm_weights(seed, l, j, H)).to(device) for j in (0, 1)]
                      for l in range(n_layers)]
        self.h0 = torch.from_numpy(residual_input(seed, M, H)).to(device)
        for io in self.io:
            io["h"] = [torch.empty((M, H), dtype=torch.float32, device=device) for _ in range(2)]
