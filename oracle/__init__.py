"""CPU oracle for TIDE's layout-aware bf16->fp32 reduce-scatter and all-gather placement.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or executes this package:
only the test suite, the smoke check and the benchmark's CPU-baseline leg use it.  It shares no
code with the HIP library (no headers, no tables, no helpers); the only thing both sides use is
the seeded input generator in ``workloads``, which contains none of the method's arithmetic.

Source of the method: the paper "The Endgame of FSDP Communication: Layout-Aware Collectives on
Copy Engines, RDMA, and NVSwitch" (arXiv 2610.38228; cited below as [Endgame]), as shown on its
abstract page and on its figures-and-tables page.  That text keeps the prose, captions and tables
but lost every math symbol, so the definitions here are the plainest reading of what survives:

* geometry  -- [Endgame] Table 2 (notation: padded per-rank rows, row length, per-rank shard
               bytes, prefix offsets, per-rank packed shard bytes) and Figure 1 (FSDP2's contract
               boundary between per-parameter tensors and flat rank-major buffers);
* reduce-scatter -- the stock FSDP2 formulation named in the abstract: pack every contributor's
               gradients into a full-group fp32 rank-major buffer, then sum the buffers.  TIDE's
               in-place path reaches the same values while skipping the pack (abstract; Table 1,
               the in-place input mode of the RS; Figure 1, every piece stored once, directly in
               its destination);
* Slot-Reuse staging -- gradients packed into an all-gather slot that is free again, then reduced from the
               slots (abstract; Figure 7); see oracle/slot.py;
* all-gather placement -- FSDP2's copy-out of the rank-major all-gather output into
               per-parameter storage (Table 7 caption: split_with_sizes_copy), which TIDE-AG
               replaces by landing shards directly (abstract; Figure 5b).

Readings where the pages are silent (each one also listed in the design notes):
  R1  padded per-rank rows m_p = ceil(rows_p / R); rank r holds rows [r*m_p, r*m_p + v) with
      v = clamp(rows_p - r*m_p, 0, m_p); the remaining (m_p - v) rows of its slice are padding.
  R2  row length L_p = product of shape_p[1:] (1 for 1-D parameters); 0-D parameters are invalid.
  R3  padding in an fp32 shard is +0.0.
  R4  contributors are summed in fixed ascending order starting from the first contributor's
      value (not from 0.0): y = x_0; y = y + x_c for c = 1..C-1, each add IEEE binary32 RNE.
  R5  bf16 -> fp32 widening is exact (the bf16 bits become the upper half of the binary32).
  R6  placement is a bit copy; padding slots of the stage are never read into a parameter.

Parity status: every function here is pinned by tests that do not retype it (brute force,
library routines, closed forms, invariants, IEEE hand-derived cases).  The pages print no values
for any result, so no pin comes from the pages' numbers; see the test modules.
"""
from .geometry import ParamGeom, group_geometry, valid_rows  # noqa: F401
from .rs import widen, pack_contributor, reduce_scatter, rs_sampled  # noqa: F401
from .ag import all_gather_place  # noqa: F401
from .brute import brute_reduce_scatter, brute_all_gather_place  # noqa: F401
from .slot import pack_slot, rs_from_slots  # noqa: F401
