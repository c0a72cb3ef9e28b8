"""GPU parity of degenerate groups: every parameter empty (S = 0), parameters of zero width (rows > 0
and a zero trailing dimension, so e_p = 0), and such parameters mixed with ordinary ones, through every
entry point (immediate, prepared and allocation-free calls, the three placement engines, Slot-Reuse)
and every launch form, against the oracle."""
import numpy as np
import pytest
import torch

import oracle
from oracle import geometry as ogeo
from all_gather_placement_amd import Launch, Layout, TIDE_AG_COPY2D, TIDE_AG_KERNEL, TIDE_AG_SDMA
from all_gather_placement_amd import tide as tb
from tests.test_gpu_parity import (POISON_BF16, assert_rs_equal, dev_bf16, host_bits_bf16, host_bits_f32,
                                   poisoned_shards, say)
from workloads import normal_bf16_bits

pytestmark = pytest.mark.gpu

CASES = [
    ([(0, 4), (0,)], 4, 3),                    # every parameter empty: S = 0, nothing to launch
    ([(5, 0), (3, 0, 2)], 3, 2),               # rows but zero width: S = 0 as well
    ([(5, 0), (9, 3), (0, 7), (1,)], 4, 5),    # degenerate parameters beside ordinary ones (with padding)
]
FORMS = [Launch.default(), Launch.bounded(2), Launch.per_cu_cap(3), Launch.cu_exclusive(2)]


def _shard_bits(shards, R, S):
    return np.stack([host_bits_f32(s) for s in shards]) if S else np.zeros((R, 0), np.uint32)


def _params(shapes):
    return [torch.full(s, POISON_BF16, dtype=torch.int16, device="cuda").view(torch.bfloat16) for s in shapes]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_degenerate_group(gpu_available, case):
    shapes, R, C = CASES[case]
    say(f"degenerate group {case}: shapes={shapes} R={R} C={C}")
    geo, S = ogeo.group_geometry(shapes, R)
    g = [[normal_bf16_bits(s, 1.0, 90 + case, c, p) for p, s in enumerate(shapes)] for c in range(C)]
    stage_bits = normal_bf16_bits((R * S,), 1.0, 95 + case, 0)
    want = oracle.reduce_scatter(g, shapes, R)
    want_ag = oracle.all_gather_place(stage_bits, shapes, R)
    want_slot = oracle.pack_slot(g[0], shapes, R)
    grads = [[dev_bf16(x) for x in row] for row in g]
    stage = dev_bf16(stage_bits)
    with Layout(shapes, R) as L:
        assert L.S == S
        L.prepare()
        for launch in FORMS:
            # immediate RS
            shards = poisoned_shards(R, S)
            L.rs_bf16_to_fp32(grads, shards, launch=launch)
            torch.cuda.synchronize()
            assert_rs_equal(_shard_bits(shards, R, S), want)
            # prepared RS, launched twice
            shards = poisoned_shards(R, S)
            call = L.bind_rs(grads, shards, launch=launch)
            call.launch()
            call.launch()
            torch.cuda.synchronize()
            call.close()
            assert_rs_equal(_shard_bits(shards, R, S), want)
            # allocation-free RS
            shards = poisoned_shards(R, S)
            tb.tide_rs_bf16_to_fp32_noalloc(L.handle, grads, shards, launch)
            torch.cuda.synchronize()
            assert_rs_equal(_shard_bits(shards, R, S), want)
            # Slot-Reuse: pack every contributor, then reduce from the slots
            if launch.form != tb.TIDE_LAUNCH_PER_CU_CAP:
                slots = [torch.full((R * S,), POISON_BF16, dtype=torch.int16, device="cuda").view(torch.bfloat16)
                         for _ in range(C)]
                for c in range(C):
                    L.slot_pack(grads[c], slots[c], launch=launch)
                torch.cuda.synchronize()
                assert np.array_equal(host_bits_bf16(slots[0]), want_slot)
                shards = poisoned_shards(R, S)
                L.rs_slots_bf16_to_fp32(slots, shards, launch=launch)
                torch.cuda.synchronize()
                assert_rs_equal(_shard_bits(shards, R, S), want)
                # placement kernel, immediate and prepared
                params = _params(shapes)
                L.ag_place(stage, params, launch=launch)
                torch.cuda.synchronize()
                for q, w in zip(params, want_ag):
                    assert np.array_equal(host_bits_bf16(q), w)
                params = _params(shapes)
                call = L.bind_ag(stage, params, launch=launch)
                call.launch()
                torch.cuda.synchronize()
                call.close()
                for q, w in zip(params, want_ag):
                    assert np.array_equal(host_bits_bf16(q), w)
        # the DMA engines and the runtime 2-D copy
        for mode in (TIDE_AG_SDMA, TIDE_AG_COPY2D):
            params = _params(shapes)
            L.ag_place(stage, params, mode=mode)
            torch.cuda.synchronize()
            for q, w in zip(params, want_ag):
                assert np.array_equal(host_bits_bf16(q), w), mode
    torch.cuda.synchronize()
