"""Slot-Reuse staging: gradients packed into an all-gather slot that is free again (oracle; test infrastructure).

In TIDE's optional Slot-Reuse mode ([Endgame] abstract; Figure 7) a contributor's gradients are first
copied into an all-gather buffer that is no longer needed, and the reduce-scatter reads them from there;
the buffer is only reused after that read.  A slot has the all-gather stage's rank-major layout (R slots of S bf16
elements, parameter p of rank r at r*S + o_p), so packing is the inverse of the all-gather copy-out:

  slot[r*S + o_p + k] = G[p].flat[r*m_p*L_p + k]   for k < v*L_p,   +0 (bits 0) for the padding.

The reduce-scatter from C slots is then the elementwise fixed-order sum of the widened slots, with the
padding forced to +0.0 (readings R3-R5), which equals the in-place reduce-scatter of the same gradients.
"""
from __future__ import annotations

import numpy as np

from .geometry import group_geometry, valid_rows
from .rs import widen


def pack_slot(grads_c, shapes, R: int) -> np.ndarray:
    """One contributor's gradients (uint16 bits, shape_p) -> flat R*S uint16 slot, padding 0."""
    geo, S = group_geometry(shapes, R)
    slot = np.zeros((R, S), dtype=np.uint16)
    for g, shape, G in zip(geo, shapes, grads_c):
        if tuple(np.shape(G)) != tuple(shape):
            raise ValueError(f"gradient shape {np.shape(G)} != parameter shape {shape}")
        rows2d = np.asarray(G, dtype=np.uint16).reshape(g.rows, g.L)
        for r in range(R):
            v = valid_rows(g.rows, g.m, r)
            if v:
                slot[r, g.o: g.o + v * g.L] = rows2d[r * g.m: r * g.m + v].ravel()
    return slot.ravel()


def rs_from_slots(slots, shapes, R: int) -> np.ndarray:
    """Reduce-scatter of C packed slots (each flat R*S uint16): (R, S) float32, padding +0.0."""
    geo, S = group_geometry(shapes, R)
    if len(slots) < 1:
        raise ValueError("need at least one contributor")
    Y = widen(np.asarray(slots[0], dtype=np.uint16).reshape(R, S)).copy()
    for s in slots[1:]:
        Y = Y + widen(np.asarray(s, dtype=np.uint16).reshape(R, S))
    for g in geo:
        for r in range(R):
            v = valid_rows(g.rows, g.m, r)
            Y[r, g.o + v * g.L: g.o + g.e] = np.float32(0.0)
    return Y
