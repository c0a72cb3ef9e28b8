"""GPU parity beyond 32-bit sizes: one parameter of more than 2^31 elements.

The work-item tables carry 64-bit element offsets and the kernels use 32-bit offsets only inside
one work item, so a parameter of (65537, 32771) bf16 elements (2,147,713,027 > 2^31; 4.3 GB per
contributor) over R = 8 ranks must reduce and place exactly like a small one.  Its rank slices
start at odd element offsets (L = 32771), the last rank holds 8186 of 8193 rows (padding), and the
source byte offsets of ranks 1..7 pass 2^31 and 2^32.  Every shard element is checked against the
oracle (from the contributor bytes read back; about 36 GB of host memory), outputs around every
2^31/2^32 boundary and segment edge once more one by one, and every element against a plain torch
fixed-order fp32 sum on the device; every placed element against the oracle's copy-out.
"""
import numpy as np
import pytest
import torch

from oracle import geometry as ogeo
from oracle import rs as ors
from all_gather_placement_amd import Launch, Layout, TIDE_AG_COPY2D, TIDE_AG_KERNEL, TIDE_AG_SDMA
from workloads import normal_bf16_cuda
from tests.test_gpu_parity import (host_bits_bf16, host_bits_f32, oracle_ag_every_element, oracle_rs_every_element,
                                   poisoned_shards, say, _locate_many)

pytestmark = pytest.mark.gpu

SHAPES = [(65537, 32771)]
R, C = 8, 2


def _boundary_positions(geo, S):
    """(r, k) shard positions whose source elements sit next to element 2^30 (byte 2^31), 3*2^29,
    element 2^31 (byte 2^32) and the start of rank 7's slice, plus each rank's first and last valid
    element and first padding element."""
    g = geo[0]
    rs, ks = [], []
    for src in (1 << 30, 3 << 29, 1 << 31, 7 * 8193 * 32771):
        for d in (-9, -8, -1, 0, 1, 7, 8, 2047, 2048, 2049):
            e = src + d
            if 0 <= e < g.rows * g.L:
                r = e // (g.m * g.L)
                rs.append(r)
                ks.append(g.o + e - r * g.m * g.L)
    for r in range(R):
        v = ogeo.valid_rows(g.rows, g.m, r)
        for k in (0, 1, v * g.L - 1, v * g.L, g.e - 1):
            if 0 <= k < S:
                rs.append(r)
                ks.append(g.o + k)
    return np.array(rs, dtype=np.int64), np.array(ks, dtype=np.int64)


@pytest.mark.timeout(900)
def test_parameter_beyond_2_31_elements(gpu_available):
    numel = SHAPES[0][0] * SHAPES[0][1]
    assert numel > (1 << 31)
    say(f"large parameter {SHAPES[0]} ({numel} elements) R={R} C={C}: generating inputs")
    torch.cuda.empty_cache()
    geo, S = ogeo.group_geometry(SHAPES, R)
    g = geo[0]
    grads = [[normal_bf16_cuda(SHAPES[0], 1.0, 200, c, 0)] for c in range(C)]
    with Layout(SHAPES, R) as L:
        assert L.S == S
        shards = poisoned_shards(R, S)
        say("large parameter: RS")
        L.rs_bf16_to_fp32(grads, shards)
        torch.cuda.synchronize()

        rng = np.random.default_rng(201)
        rs_b, ks_b = _boundary_positions(geo, S)
        rs_ = np.concatenate([rs_b, rng.integers(0, R, 4000)])
        ks = np.concatenate([ks_b, rng.integers(0, S, 4000)])
        _, src = _locate_many(geo, R, rs_, ks)
        got = np.empty(len(rs_), dtype=np.uint32)
        for r in range(R):
            sel = np.nonzero(rs_ == r)[0]
            if sel.size:
                got[sel] = host_bits_f32(shards[r][torch.from_numpy(ks[sel]).cuda()])
        vals = np.zeros((C, len(rs_)), dtype=np.uint16)
        sel = np.nonzero(src >= 0)[0]
        idx = torch.from_numpy(src[sel]).cuda()
        for c in range(C):
            vals[c, sel] = host_bits_bf16(grads[c][0].reshape(-1)[idx])
        want = np.where(src >= 0, ors.rs_sampled(vals).view(np.uint32), 0).astype(np.uint32)
        assert np.array_equal(got, want), f"{int((got != want).sum())} sampled mismatches"
        say(f"large parameter: {len(rs_)} sampled outputs OK")

        oracle_rs_every_element(SHAPES, R, geo, grads, shards, "large parameter")
        say("large parameter: every element equal to the oracle")

        acc = grads[0][0].reshape(-1).float()
        for c in range(1, C):
            acc += grads[c][0].reshape(-1).float()
        for r in range(R):
            v = ogeo.valid_rows(g.rows, g.m, r)
            seg = shards[r][g.o: g.o + g.e]
            lo, hi = r * g.m * g.L, (r * g.m + v) * g.L
            assert torch.equal(seg[: v * g.L].view(torch.int32), acc[lo:hi].view(torch.int32)), r
            assert bool((seg[v * g.L:].view(torch.int32) == 0).all()), r
        del acc
        say("large parameter: torch fixed-order sum equal")

        # the CU-exclusive launch (one launch, 64-bit item and element offsets) gives the same shards
        say("large parameter: RS, CU-exclusive workgroups of 4 items")
        shards_x = poisoned_shards(R, S)
        L.rs_bf16_to_fp32(grads, shards_x, launch=Launch.cu_exclusive(4))
        torch.cuda.synchronize()
        for r in range(R):
            assert torch.equal(shards_x[r].view(torch.int32), shards[r].view(torch.int32)), r
        del grads, shards, shards_x
        torch.cuda.empty_cache()

        stage = normal_bf16_cuda((R * S,), 1.0, 202, 0)
        want_p = None
        for mode, launch in ((TIDE_AG_KERNEL, Launch()), (TIDE_AG_SDMA, Launch()), (TIDE_AG_COPY2D, Launch()),
                             (TIDE_AG_KERNEL, Launch.cu_exclusive(4))):
            say(f"large parameter: AG mode={mode} launch={launch}")
            param = torch.full(SHAPES[0], float("nan"), dtype=torch.bfloat16, device="cuda")
            L.ag_place(stage, [param], mode=mode, launch=launch)
            torch.cuda.synchronize()
            want_p = oracle_ag_every_element(SHAPES, R, stage, [param], f"large parameter AG mode={mode}", want_p)
            del param
        say("large parameter: AG every element equal to the oracle (all engines)")
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
