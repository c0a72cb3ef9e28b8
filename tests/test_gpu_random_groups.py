"""Randomised GPU parity: many small seeded groups, each checked bit for bit against the oracle.

Every group draws R, C (1-12; 13-40 in a second set, which reaches the runtime-C kernels and
explicit per-CU caps), the parameter shapes (1-3 dimensions, rows 0-3000, so empty parameters,
rows < R and ragged tails all occur), a launch form and per-buffer base offsets (0-7 elements, so
both the vector and the element paths run), then runs the reduce-scatter, the placement and the
Slot-Reuse packing through the C ABI.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import geometry as ogeo
from all_gather_placement_amd import Launch, Layout
from tests.test_gpu_parity import POISON_BF16, assert_rs_equal, dev_bf16, host_bits_bf16, host_bits_f32, poisoned_shards, say

pytestmark = pytest.mark.gpu

N_GROUPS = 40


def _random_group(rng, c_lo=1, c_hi=13):
    R = int(rng.integers(1, 18))
    C = int(rng.integers(c_lo, c_hi))
    shapes = []
    for _ in range(int(rng.integers(1, 6))):
        nd = int(rng.integers(1, 4))
        rows = int(rng.choice([0, int(rng.integers(1, R + 1)), int(rng.integers(1, 3001))]))
        rest = [int(rng.integers(1, 40)) for _ in range(nd - 1)]
        while rows * int(np.prod(rest, dtype=np.int64)) > 200_000:
            rows //= 2
        shapes.append(tuple([rows] + rest))
    budget = int(rng.choice([0, 0, 1, 2, 5, 64]))
    return shapes, R, C, Launch.bounded(budget) if budget else Launch.default()


def _random_inputs(rng, shapes, R, C, S):
    """Random bf16 bit patterns with the exponent's top bit cleared: every finite value below 2 in
    magnitude, subnormals and signed zeros included (no inf or NaN, so results compare bit for bit)."""
    bits = lambda size: np.asarray(rng.integers(0, 1 << 16, size=size), dtype=np.uint16) & np.uint16(0xBFFF)
    return [[bits(s) for s in shapes] for _ in range(C)], bits(R * S)


@pytest.mark.parametrize("case", range(N_GROUPS))
def test_random_group_bit_exact(gpu_available, case):
    rng = np.random.default_rng(1000 + case)
    shapes, R, C, launch = _random_group(rng)
    _check_group(rng, case, shapes, R, C, launch, launch)


@pytest.mark.parametrize("case", range(12))
def test_random_group_many_contributors(gpu_available, case):
    """C from 13 to 40: the largest compiled contributor counts and the runtime-C kernels, with
    the default, bounded launches and explicit per-CU caps."""
    rng = np.random.default_rng(5000 + case)
    shapes, R, C, launch = _random_group(rng, 13, 41)
    cap = int(rng.choice([0, 1, 3, 64]))
    _check_group(rng, case, shapes, R, C, Launch.per_cu_cap(cap) if cap else launch, launch)


@pytest.mark.parametrize("case", range(16))
def test_random_group_cu_exclusive(gpu_available, case):
    """The CU-exclusive RS (1 .. 8 items per CU-wide workgroup, and 16 where C allows two items per
    group) on random groups, C 1-12 and 13-40 in turn (compiled and runtime-C forms),
    misaligned bases in a third of them; the placement and the packing in the same form in every
    other group."""
    rng = np.random.default_rng(7000 + case)
    shapes, R, C, launch = _random_group(rng, *((1, 13) if case % 2 == 0 else (13, 41)))
    ag_launch = Launch.cu_exclusive(1 + (3 * case) % 8) if case % 4 < 2 else launch
    n = 1 + case % 8
    if case % 4 == 0 and C <= 4:
        n = 16
    _check_group(rng, case, shapes, R, C, Launch.cu_exclusive(n), ag_launch)


def _check_group(rng, case, shapes, R, C, rs_launch, ag_launch):
    offset = (lambda: int(rng.integers(0, 8))) if case % 3 == 0 else (lambda: 0)
    say(f"random group {case}: shapes={shapes} R={R} C={C} launch rs={rs_launch} ag={ag_launch} "
        f"offsets={'on' if case % 3 == 0 else 'off'}")
    geo, S = ogeo.group_geometry(shapes, R)
    g, stage_bits = _random_inputs(rng, shapes, R, C, S)
    want = oracle.reduce_scatter(g, shapes, R)
    want_ag = oracle.all_gather_place(stage_bits, shapes, R)
    with Layout(shapes, R) as L:
        grads = [[dev_bf16(x, offset()) for x in row] for row in g]
        shards = poisoned_shards(R, S, offset())
        L.rs_bf16_to_fp32(grads, shards, launch=rs_launch)
        stage = dev_bf16(stage_bits, offset())
        params = []
        for s in shapes:
            n = int(np.prod(s, dtype=np.int64))
            o = offset()
            buf = torch.full((n + o + 8,), POISON_BF16, dtype=torch.int16, device="cuda")
            params.append(buf[o: o + n].view(torch.bfloat16).reshape(s))
        L.ag_place(stage, params, launch=ag_launch)
        o = offset()
        slot_buf = torch.full((R * S + o + 8,), POISON_BF16, dtype=torch.int16, device="cuda")
        slot = slot_buf[o: o + R * S].view(torch.bfloat16)
        L.slot_pack(grads[0], slot, launch=ag_launch)
        torch.cuda.synchronize()
        got = np.stack([host_bits_f32(x) for x in shards]) if S else np.zeros((R, 0), np.uint32)
        assert_rs_equal(got, want)
        for q, w in zip(params, want_ag):
            assert np.array_equal(host_bits_bf16(q), w)
        assert np.array_equal(host_bits_bf16(slot), oracle.pack_slot(g[0], shapes, R))
