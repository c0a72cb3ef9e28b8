"""Scalar brute-force formulations, for tiny groups only (oracle; test infrastructure).

A second, element-at-a-time statement of the same results as :mod:`oracle.rs` and
:mod:`oracle.ag`, written from the element's point of view rather than the pack's: for output
element (r, p, i, j) -- row i of rank r's slice of parameter p, column j -- the global row is
g = r*m_p + i; the element is padding (+0.0 / not placed) when g >= rows_p, otherwise the
fixed-order fp32 sum over contributors of G[c][p][g, j] (readings R1-R5).  Pure Python loops with
numpy float32 scalars; only for groups of a few hundred elements.
"""
from __future__ import annotations

import numpy as np

from .geometry import group_geometry


def _bf16_scalar(bits: int) -> np.float32:
    return np.array([int(bits) << 16], dtype=np.uint32).view(np.float32)[0]


def brute_reduce_scatter(grads, shapes, R: int) -> np.ndarray:
    geo, S = group_geometry(shapes, R)
    C = len(grads)
    out = np.full((R, S), np.nan, dtype=np.float32)
    for r in range(R):
        for p, g in enumerate(geo):
            for i in range(g.m):
                grow = r * g.m + i
                for j in range(g.L):
                    k = g.o + i * g.L + j
                    if grow >= g.rows:
                        out[r, k] = np.float32(0.0)
                        continue
                    acc = None
                    for c in range(C):
                        x = _bf16_scalar(np.asarray(grads[c][p]).reshape(g.rows, g.L)[grow, j])
                        acc = x if acc is None else np.float32(acc + x)
                    out[r, k] = acc
    return out


def brute_all_gather_place(stage_bits, shapes, R: int):
    geo, S = group_geometry(shapes, R)
    st = np.asarray(stage_bits, dtype=np.uint16).ravel()
    params = []
    for p, (g, shape) in enumerate(zip(geo, shapes)):
        flat = np.zeros(g.rows * g.L, dtype=np.uint16)
        for grow in range(g.rows):
            r, i = divmod(grow, g.m)
            for j in range(g.L):
                flat[grow * g.L + j] = st[r * S + g.o + i * g.L + j]
        params.append(flat.reshape(shape))
    return params
