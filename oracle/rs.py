"""Reduce-scatter of bf16 per-parameter gradients into R flat fp32 shards (oracle; test infra).

The result is defined by the stock FSDP2 formulation that [Endgame]'s abstract describes (and
Table 8's caption, whose FSDP2 columns include the full-group pack): every contributor's
per-parameter gradients are packed into one full-group fp32 buffer laid out rank-major (R slots of
S elements, parameter p of slot r at offset o_p, padding zero), and the packed buffers of the C
contributors are summed elementwise; slot r of the sum is rank r's fp32 shard.  TIDE's in-place
reduce-scatter (abstract; Figure 6a, node-local fp32 sums; Table 1, in-place input) computes the
same values without the pack, which is why this formulation serves as the definition.

Summation order (reading R4): y = x_0, then y = y + x_c for c = 1..C-1, each add one numpy float32
elementwise add (IEEE binary32, round to nearest even).  No library reduction over the contributor
axis is used, because its order is the library's choice.
"""
from __future__ import annotations

import numpy as np

from .geometry import group_geometry, valid_rows


def widen(bits: np.ndarray) -> np.ndarray:
    """bf16 bits (uint16) -> float32, exactly: the 16 bits become the binary32's upper half (R5)."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def pack_contributor(grads_c, shapes, R: int) -> np.ndarray:
    """Stock full-group pack of one contributor: (R, S) float32, rank-major, padding +0.0 (R3)."""
    geo, S = group_geometry(shapes, R)
    X = np.zeros((R, S), dtype=np.float32)
    for g, shape, G in zip(geo, shapes, grads_c):
        if tuple(np.shape(G)) != tuple(shape):
            raise ValueError(f"gradient shape {np.shape(G)} != parameter shape {shape}")
        rows2d = np.asarray(G, dtype=np.uint16).reshape(g.rows, g.L)
        for r in range(R):
            v = valid_rows(g.rows, g.m, r)
            if v == 0:
                continue
            piece = rows2d[r * g.m: r * g.m + v].ravel()
            X[r, g.o: g.o + v * g.L] = widen(piece)
    return X


def reduce_scatter(grads, shapes, R: int) -> np.ndarray:
    """RS of C contributors' gradients ``grads[c][p]`` (uint16 bits): returns shards as (R, S) f32.

    Pack each contributor (stock formulation), then add the packs in ascending contributor order.
    """
    C = len(grads)
    if C < 1:
        raise ValueError("need at least one contributor")
    Y = pack_contributor(grads[0], shapes, R)
    for c in range(1, C):
        Y = Y + pack_contributor(grads[c], shapes, R)
    return Y


def rs_sampled(values_by_contributor: np.ndarray) -> np.ndarray:
    """Fixed-order fp32 sum of already-gathered bf16 inputs, one output per column.

    ``values_by_contributor`` is (C, n) uint16: column j holds the C contributors' bf16 inputs of one
    sampled output element.  Used to check individual outputs of full-size runs, where the whole
    pack would not fit the host.  Same order and rounding as :func:`reduce_scatter` (R4, R5).
    """
    V = np.asarray(values_by_contributor, dtype=np.uint16)
    y = widen(V[0]).copy()
    for c in range(1, V.shape[0]):
        y = y + widen(V[c])
    return y


def locate(shapes, R: int, r: int, k: int):
    """Where output element k of shard r comes from: (p, flat source index or None for padding)."""
    geo, S = group_geometry(shapes, R)
    if not (0 <= r < R and 0 <= k < S):
        raise IndexError("output element out of range")
    for p, g in enumerate(geo):
        if g.o <= k < g.o + g.e:
            j = k - g.o
            v = valid_rows(g.rows, g.m, r)
            if j < v * g.L:
                return p, r * g.m * g.L + j
            return p, None
    raise AssertionError("unreachable: offsets cover [0, S)")
