"""GPU parity of the Slot-Reuse path (pack into an all-gather slot that is free again, reduce from the slots).

Packing is compared bit for bit with the oracle's pack (padding must become +0 whatever the slot
held); the reduce-scatter from slots with the oracle's slot reduction (padding in the slots is
poisoned and must be ignored); and at full size the whole Slot-Reuse chain must reproduce the
in-place reduce-scatter bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import geometry as ogeo
from all_gather_placement_amd import Launch, Layout
from workloads import ORDERED, TINY, normal_bf16_bits, normal_bf16_cuda
from tests.test_gpu_parity import GROUPS, POISON_BF16, assert_rs_equal, dev_bf16, host_bits_bf16, host_bits_f32, poisoned_shards, say

pytestmark = pytest.mark.gpu


def poisoned_slot(R, S, pad_elems=0):
    buf = torch.full((R * S + pad_elems + 8,), POISON_BF16, dtype=torch.int16, device="cuda")
    return buf[pad_elems: pad_elems + R * S].view(torch.bfloat16)


@pytest.mark.parametrize("case", range(len(GROUPS)))
def test_slot_pack_bit_exact(gpu_available, case):
    shapes, R, C = GROUPS[case]
    say(f"slot pack group {case}")
    g = [normal_bf16_bits(s, 1.0, 90 + case, 0, p) for p, s in enumerate(shapes)]
    geo, S = ogeo.group_geometry(shapes, R)
    want = oracle.pack_slot(g, shapes, R)
    with Layout(shapes, R) as L:
        for launch in (Launch.default(), Launch.bounded(3), Launch.cu_exclusive(6)):
            slot = poisoned_slot(R, S)
            L.slot_pack([dev_bf16(x) for x in g], slot, launch=launch)
            torch.cuda.synchronize()
            assert np.array_equal(host_bits_bf16(slot), want)


@pytest.mark.parametrize("g_off,s_off", [(1, 0), (0, 3), (5, 5), (2, 7)])
def test_slot_pack_alignment(gpu_available, g_off, s_off):
    shapes, R = [(300, 17), (1025,), (8, 64), (5, 3)], 4
    say(f"slot pack alignment g_off={g_off} s_off={s_off}")
    g = [normal_bf16_bits(s, 1.0, 91, 0, p) for p, s in enumerate(shapes)]
    geo, S = ogeo.group_geometry(shapes, R)
    with Layout(shapes, R) as L:
        for launch in (Launch.default(), Launch.bounded(3)):
            slot = poisoned_slot(R, S, s_off)
            L.slot_pack([dev_bf16(x, (g_off * (p + 1)) % 8) for p, x in enumerate(g)], slot, launch=launch)
            torch.cuda.synchronize()
            assert np.array_equal(host_bits_bf16(slot), oracle.pack_slot(g, shapes, R)), launch


@pytest.mark.parametrize("case", range(len(GROUPS)))
def test_rs_from_slots_bit_exact(gpu_available, case):
    shapes, R, C = GROUPS[case]
    say(f"rs from slots group {case}")
    geo, S = ogeo.group_geometry(shapes, R)
    g = [[normal_bf16_bits(s, 1.0, 92 + case, c, p) for p, s in enumerate(shapes)] for c in range(C)]
    slots_bits = []
    for c in range(C):
        sb = oracle.pack_slot(g[c], shapes, R).reshape(R, S)
        for gg in geo:  # garbage in the padding: the reduction must ignore it
            for r in range(R):
                v = ogeo.valid_rows(gg.rows, gg.m, r)
                sb[r, gg.o + v * gg.L: gg.o + gg.e] = POISON_BF16
        slots_bits.append(sb.ravel())
    want = oracle.rs_from_slots(slots_bits, shapes, R)
    assert np.array_equal(want.view(np.uint32), oracle.reduce_scatter(g, shapes, R).view(np.uint32))
    with Layout(shapes, R) as L:
        forms = [Launch.default(), Launch.bounded(5), Launch.per_cu_cap(4), Launch.cu_exclusive(2)]
        forms += [Launch.cu_exclusive(16)] if C <= 4 else []
        for launch in forms:
            shards = poisoned_shards(R, S)
            L.rs_slots_bf16_to_fp32([dev_bf16(x) for x in slots_bits], shards, launch=launch)
            torch.cuda.synchronize()
            assert_rs_equal(np.stack([host_bits_f32(x) for x in shards]), want)


@pytest.mark.parametrize("C", [5, 20])
def test_rs_from_slots_unaligned(gpu_available, C):
    shapes, R = [(300, 17), (1025,), (8, 64)], 4
    say(f"rs from slots, unaligned bases, C={C}")
    geo, S = ogeo.group_geometry(shapes, R)
    g = [[normal_bf16_bits(s, 1.0, 93, c, p) for p, s in enumerate(shapes)] for c in range(C)]
    slots_bits = [oracle.pack_slot(g[c], shapes, R) for c in range(C)]
    with Layout(shapes, R) as L:
        shards = poisoned_shards(R, S, 1)
        L.rs_slots_bf16_to_fp32([dev_bf16(x, c % 8) for c, x in enumerate(slots_bits)], shards)
        torch.cuda.synchronize()
        assert_rs_equal(np.stack([host_bits_f32(x) for x in shards]), oracle.reduce_scatter(g, shapes, R))


def test_slot_reuse_chain_on_one_stream(gpu_available):
    """Pack every contributor into its slot, then reduce from the slots, no host sync in between."""
    say("slot reuse chain, tiny")
    geo, S = ogeo.group_geometry(TINY.shapes, TINY.R)
    g = [[normal_bf16_bits(s, TINY.sigma, TINY.cfg_id, c, p) for p, s in enumerate(TINY.shapes)] for c in range(TINY.C)]
    grads = [[dev_bf16(x) for x in row] for row in g]
    with Layout(TINY.shapes, TINY.R) as L:
        slots = [poisoned_slot(TINY.R, S) for _ in range(TINY.C)]
        shards = poisoned_shards(TINY.R, S)
        torch.cuda.synchronize()
        for c in range(TINY.C):
            L.slot_pack(grads[c], slots[c])
        L.rs_slots_bf16_to_fp32(slots, shards)
        torch.cuda.synchronize()
        assert_rs_equal(np.stack([host_bits_f32(x) for x in shards]), oracle.reduce_scatter(g, TINY.shapes, TINY.R))


@pytest.mark.parametrize("cfg", [c for c in ORDERED if c.name != "tiny"], ids=lambda c: c.name)
def test_full_size_slot_reuse_equals_in_place(gpu_available, cfg):
    say(f"full size slot reuse {cfg.name}")
    torch.cuda.empty_cache()
    geo, S = ogeo.group_geometry(cfg.shapes, cfg.R)
    with Layout(cfg.shapes, cfg.R) as L:
        grads = [[normal_bf16_cuda(s, cfg.sigma, cfg.cfg_id, c, p) for p, s in enumerate(cfg.shapes)]
                 for c in range(cfg.C)]
        ref = poisoned_shards(cfg.R, S)
        L.rs_bf16_to_fp32(grads, ref)
        slots = []
        for c in range(cfg.C):
            slot = poisoned_slot(cfg.R, S)
            L.slot_pack(grads[c], slot)
            slots.append(slot)
        torch.cuda.synchronize()
        # each packed slot, placed back, is the contributor's gradients (bit for bit)
        params = [torch.empty(s, dtype=torch.bfloat16, device="cuda") for s in cfg.shapes]
        L.ag_place(slots[cfg.C - 1], params)
        torch.cuda.synchronize()
        for p in range(cfg.P):
            assert torch.equal(params[p].view(torch.int16), grads[cfg.C - 1][p].view(torch.int16)), p
        del params, grads
        out = poisoned_shards(cfg.R, S)
        L.rs_slots_bf16_to_fp32(slots, out)
        torch.cuda.synchronize()
        for r in range(cfg.R):
            assert torch.equal(out[r].view(torch.int32), ref[r].view(torch.int32)), r
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
