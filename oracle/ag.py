"""All-gather placement: rank-major bf16 stage -> per-parameter storage (oracle; test infra).

[Endgame] Figure 1 puts FSDP2's contract boundary between the flat rank-major all-gather output
and per-parameter storage; stock FSDP2 converts with a copy-out (Table 7's caption names its fused
split_with_sizes_copy), and TIDE-AG lands each rank's piece straight into parameter storage,
filling each parameter by a single strided copy (Figure 5b; abstract).  Both give the same parameter contents,
defined here as the copy-out:

  stage viewed as (R, S); take columns [o_p, o_p + e_p) -> (R, m_p, L_p) -> (R*m_p, L_p);
  keep the first rows_p rows (the rest are padding, reading R6); reshape to shape_p.

The stage is handled as uint16 bits, so the copy is exact for every pattern (NaNs included).
"""
from __future__ import annotations

import numpy as np

from .geometry import group_geometry


def all_gather_place(stage_bits: np.ndarray, shapes, R: int):
    """Return the P parameter tensors (uint16 bits, shape_p) placed from a flat R*S stage."""
    geo, S = group_geometry(shapes, R)
    st = np.asarray(stage_bits, dtype=np.uint16)
    if st.size != R * S:
        raise ValueError(f"stage has {st.size} elements, expected R*S = {R * S}")
    st = st.reshape(R, S)
    out = []
    for g, shape in zip(geo, shapes):
        block = st[:, g.o: g.o + g.e].reshape(R * g.m, g.L)
        out.append(block[: g.rows].reshape(shape).copy())
    return out
