"""Row-sharded, per-rank-padded geometry of one FSDP parameter group (oracle; test infrastructure).

[Endgame] Table 2 names, per parameter p of a group of P parameters sharded over R ranks: its
padded per-rank rows and row length, its per-rank shard bytes and prefix offset, and the group's
per-rank packed shard bytes.  The symbols were lost in extraction; the names used here:

  rows_p  dim 0 of parameter p
  L_p     row length = product of the remaining dims (1 for a 1-D parameter)       (reading R2)
  m_p     padded per-rank rows = ceil(rows_p / R)                                 (reading R1)
  e_p     per-rank shard elements = m_p * L_p   (bytes: x2 in a bf16 buffer, x4 in fp32)
  o_p     prefix offset = sum of e_q over q < p, in elements
  S       per-rank packed shard elements = sum of e_p
  v(p,r)  rows of parameter p that rank r really holds = clamp(rows_p - r*m_p, 0, m_p)
"""
from __future__ import annotations

from dataclasses import dataclass


@dataclass(frozen=True)
class ParamGeom:
    rows: int
    L: int
    m: int
    e: int
    o: int


def valid_rows(rows: int, m: int, r: int) -> int:
    """v(p, r): rows of the parameter that rank r holds before its padding (reading R1)."""
    return max(0, min(m, rows - r * m))


def param_rows_len(shape) -> tuple[int, int]:
    """(rows_p, L_p) of one parameter shape (reading R2)."""
    shape = tuple(int(d) for d in shape)
    if len(shape) == 0:
        raise ValueError("0-d parameters have no row dimension")
    if any(d < 0 for d in shape):
        raise ValueError("negative dimension")
    L = 1
    for d in shape[1:]:
        L *= d
    return shape[0], L


def group_geometry(shapes, R: int):
    """Per-parameter geometry and S for parameters ``shapes`` (storage order) over R ranks."""
    if R < 1:
        raise ValueError("R must be >= 1")
    geo = []
    o = 0
    for shape in shapes:
        rows, L = param_rows_len(shape)
        m = -(-rows // R)  # ceil
        e = m * L
        geo.append(ParamGeom(rows=rows, L=L, m=m, e=e, o=o))
        o += e
    return geo, o
