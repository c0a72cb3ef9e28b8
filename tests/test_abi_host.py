"""Host-only tests of the C-ABI library (no GPU, no compute calls).

* the library loads and exports every function that include/tide.h declares;
* layout geometry equals the oracle's independent geometry on every workload and on random tiny
  groups;
* the work-item tables tile every shard element and every placed parameter element exactly once,
  and every kernel access they imply stays inside its buffer (checked here, before any launch);
* argument validation returns TIDE_ERR_INVALID before any HIP call.
"""
import ctypes
import os
import re

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import all_gather_placement_amd as tide
from all_gather_placement_amd import tide as tb
from oracle import geometry as ogeo
from workloads import ORDERED, TINY

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "tide.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = set(re.findall(r"\b(tide_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_library_exports_every_declared_symbol():
    lib = tb.load_library()
    names = _declared_functions()
    assert "tide_rs_bf16_to_fp32" in names and "tide_ag_place" in names and "tide_layout_create" in names
    for n in names:
        assert hasattr(lib, n), f"{n} declared in include/tide.h but not exported"
    # and the binding exposes the three entry points under the same names
    for n in ("tide_layout_create", "tide_rs_bf16_to_fp32", "tide_ag_place"):
        assert callable(getattr(tide, n))


def test_status_strings():
    lib = tb.load_library()
    assert lib.tide_status_str(0) == b"TIDE_OK"
    assert lib.tide_status_str(1) == b"TIDE_ERR_INVALID"
    assert lib.tide_status_str(4) == b"TIDE_ERR_UNSUPPORTED"
    assert lib.tide_status_str(99) == b"unknown"
    assert lib.tide_last_hip_error() == 0


def _check_geometry(shapes, R):
    geo, S = ogeo.group_geometry(shapes, R)
    with tide.Layout(shapes, R) as L:
        assert L.S == S and L.P == len(shapes)
        for p, g in enumerate(geo):
            assert L.param(p) == (g.rows, g.L, g.m, g.o)
            for r in range(R):
                v = ogeo.valid_rows(g.rows, g.m, r)
                assert L.segment(p, r) == (r * g.m * g.L, v * g.L, g.o, (g.m - v) * g.L)


@pytest.mark.parametrize("cfg", ORDERED, ids=lambda c: c.name)
def test_layout_geometry_matches_oracle(cfg):
    if cfg.P > 50:
        # segment queries over 391 x 16 are fine but slow through ctypes; sample them
        geo, S = ogeo.group_geometry(cfg.shapes, cfg.R)
        with tide.Layout(cfg.shapes, cfg.R) as L:
            assert L.S == S
            for p in list(range(0, cfg.P, 37)) + [cfg.P - 1]:
                g = geo[p]
                assert L.param(p) == (g.rows, g.L, g.m, g.o)
        return
    _check_geometry(cfg.shapes, cfg.R)


@st.composite
def groups(draw):
    R = draw(st.integers(1, 70))
    P = draw(st.integers(1, 6))
    shapes = []
    for _ in range(P):
        nd = draw(st.integers(1, 4))
        rows = draw(st.integers(0, 300))
        rest = [draw(st.integers(0, 9)) for _ in range(nd - 1)]
        shapes.append(tuple([rows] + rest))
    return shapes, R


@settings(max_examples=80, deadline=None)
@given(groups())
def test_layout_geometry_hypothesis(g):
    shapes, R = g
    _check_geometry(shapes, R)


def library_item_sizes():
    """(RS, AG) work-item lengths of the built library, read from a layout of one 2^20-element
    parameter on one rank: every item of an aligned segment is full."""
    with tide.Layout([(1 << 20,)], 1) as L:
        n_rs, n_ag = L.num_rs_chunks, L.num_ag_chunks
    assert (1 << 20) % n_rs == 0 and (1 << 20) % n_ag == 0
    return (1 << 20) // n_rs, (1 << 20) // n_ag


def check_items_tile_exactly(shapes, R, rs_items, ag_items, rs_chunk=None, ag_chunk=None):
    """Every shard element written once, every parameter element placed once, all in bounds;
    inside a segment every item but the first and the last is a full one."""
    if rs_chunk is None:
        rs_chunk, ag_chunk = library_item_sizes()
    geo, S = ogeo.group_geometry(shapes, R)
    numel = [g.rows * g.L for g in geo]
    # --- RS: bounds
    p, r, src, dst, nv, npad = (rs_items[:, i] for i in range(6))
    assert np.all((p >= 0) & (p < len(shapes)) & (r >= 0) & (r < R))
    assert np.all((nv >= 0) & (npad >= 0) & (nv + npad > 0) & (nv <= rs_chunk) & (npad <= rs_chunk))
    assert np.all(dst >= 0) and np.all(dst + nv + npad <= S)
    nz = nv > 0
    numel_p = np.array(numel, dtype=np.int64)[p]
    assert np.all(src[nz] >= 0) and np.all(src[nz] + nv[nz] <= numel_p[nz])
    # --- RS: each (r, k) written once; valid outputs read the right source element
    cover = np.zeros((R, S), dtype=np.int32)
    for i in range(len(rs_items)):
        cover[r[i], dst[i]: dst[i] + nv[i] + npad[i]] += 1
    assert np.all(cover == 1)
    for q, g in enumerate(geo):
        for rr in range(R):
            v = ogeo.valid_rows(g.rows, g.m, rr)
            sel = (p == q) & (r == rr) & nz
            # valid items of this segment are contiguous in both spaces with the same offset delta
            assert np.all(src[sel] - r[sel] * g.m * g.L == dst[sel] - g.o)
            assert int(nv[sel].sum()) == v * g.L
            assert int(npad[(p == q) & (r == rr)].sum()) == (g.m - v) * g.L
            inner = np.sort(src[sel])[1:-1]
            assert np.all(nv[sel][np.argsort(src[sel])][1:-1] == rs_chunk), "interior items are full"
            assert np.all((inner - (rr * g.m * g.L) // 8 * 8) % rs_chunk == 0)
    # interior item boundaries on 16-byte (8-element) source boundaries
    starts_inside = nz & (src % 8 != 0)
    for i in np.nonzero(starts_inside)[0]:
        q, rr = p[i], r[i]
        assert src[i] == rr * geo[q].m * geo[q].L, "only a segment's first item may start unaligned"
    # --- AG
    if len(ag_items):
        ap, asrc, adst, an = (ag_items[:, i] for i in range(4))
        assert np.all((an > 0) & (an <= ag_chunk))
        assert np.all(asrc >= 0) and np.all(asrc + an <= R * S)
        anumel = np.array(numel, dtype=np.int64)[ap]
        assert np.all(adst >= 0) and np.all(adst + an <= anumel)
        for q, g in enumerate(geo):
            pc = np.zeros(numel[q], dtype=np.int32)
            for i in np.nonzero(ap == q)[0]:
                pc[adst[i]: adst[i] + an[i]] += 1
                # stage slot rank and the destination row agree
                rr = asrc[i] // S
                assert asrc[i] - rr * S - g.o == adst[i] - rr * g.m * g.L
                assert 0 <= asrc[i] - rr * S - g.o and asrc[i] - rr * S - g.o + an[i] <= g.e
            assert np.all(pc == 1)
    else:
        assert sum(numel) == 0


def check_slot_items_tile(shapes, R, ag_items, pad_items):
    """A packed slot: AG items (valid parts) and padding items cover [0, R*S) exactly once."""
    geo, S = ogeo.group_geometry(shapes, R)
    cover = np.zeros(R * S, dtype=np.int32)
    for src, n in zip(ag_items[:, 1], ag_items[:, 3]):
        cover[src: src + n] += 1
    for off, n in pad_items:
        assert 0 <= off and off + n <= R * S
        cover[off: off + n] += 1
    assert np.all(cover == 1)


@settings(max_examples=60, deadline=None)
@given(groups())
def test_work_items_tile_hypothesis(g):
    shapes, R = g
    with tide.Layout(shapes, R) as L:
        check_items_tile_exactly(shapes, R, L.rs_items(), L.ag_items())
        check_slot_items_tile(shapes, R, L.ag_items(), L.slot_pad_items())


def test_work_items_tile_tiny():
    with tide.Layout(TINY.shapes, TINY.R) as L:
        check_items_tile_exactly(TINY.shapes, TINY.R, L.rs_items(), L.ag_items())
        check_slot_items_tile(TINY.shapes, TINY.R, L.ag_items(), L.slot_pad_items())
        assert int(L.slot_pad_items()[:, 1].sum()) == 32


@pytest.mark.parametrize("cfg", [c for c in ORDERED if c.name != "tiny"], ids=lambda c: c.name)
def test_work_items_full_configs_in_bounds(cfg):
    """Full workloads: bounds and exact coverage, checked with interval sums (no dense arrays)."""
    geo, S = ogeo.group_geometry(cfg.shapes, cfg.R)
    with tide.Layout(cfg.shapes, cfg.R) as L:
        it = L.rs_items()
        ag = L.ag_items()
    p, r, src, dst, nv, npad = (it[:, i] for i in range(6))
    numel = np.array([g.rows * g.L for g in geo], dtype=np.int64)
    assert np.all(src >= 0) and np.all(src + nv <= numel[p])
    assert np.all(dst >= 0) and np.all(dst + nv + npad <= S)
    # per shard: items sorted by dst tile [0, S) with no gap or overlap
    for rr in range(cfg.R):
        sel = r == rr
        order = np.argsort(dst[sel])
        d = dst[sel][order]
        n = (nv + npad)[sel][order]
        assert d[0] == 0 and np.all(d[1:] == d[:-1] + n[:-1]) and d[-1] + n[-1] == S
    # every source element of every parameter is read by exactly one item
    assert int(nv.sum()) == cfg.numel()
    # all large workloads are 16-byte aligned everywhere: the vector path covers everything
    assert np.all(src % 8 == 0) and np.all(dst % 4 == 0)
    ap, asrc, adst, an = (ag[:, i] for i in range(4))
    assert np.all(asrc + an <= cfg.R * S) and np.all(adst + an <= numel[ap])
    assert int(an.sum()) == cfg.numel()
    assert np.all((asrc - adst) % 8 == 0)


# ------------------------------------------------------------------------------------------------
# Argument validation: every case returns before any HIP call
# ------------------------------------------------------------------------------------------------

def _vp_array(vals):
    return (ctypes.c_void_p * max(len(vals), 1))(*vals)


def test_layout_create_rejects_bad_arguments():
    lib = tb.load_library()
    out = ctypes.c_void_p()
    nd = (ctypes.c_int32 * 1)(2)
    dims = (ctypes.c_int64 * 2)(4, 4)
    assert lib.tide_layout_create(0, nd, dims, 4, ctypes.byref(out)) == tb.TIDE_ERR_INVALID
    assert lib.tide_layout_create(1, nd, dims, 0, ctypes.byref(out)) == tb.TIDE_ERR_INVALID
    assert lib.tide_layout_create(1, None, dims, 4, ctypes.byref(out)) == tb.TIDE_ERR_INVALID
    assert lib.tide_layout_create(1, nd, dims, 4, None) == tb.TIDE_ERR_INVALID
    nd0 = (ctypes.c_int32 * 1)(0)
    assert lib.tide_layout_create(1, nd0, dims, 4, ctypes.byref(out)) == tb.TIDE_ERR_INVALID
    neg = (ctypes.c_int64 * 2)(4, -1)
    assert lib.tide_layout_create(1, nd, neg, 4, ctypes.byref(out)) == tb.TIDE_ERR_INVALID
    huge = (ctypes.c_int64 * 2)(1 << 40, 1 << 40)
    assert lib.tide_layout_create(1, nd, huge, 4, ctypes.byref(out)) == tb.TIDE_ERR_INVALID
    assert out.value is None
    assert lib.tide_layout_num_params(None) == -1 and lib.tide_layout_shard_numel(None) == -1
    lib.tide_layout_destroy(None)


def test_query_rejects_out_of_range():
    lib = tb.load_library()
    with tide.Layout(TINY.shapes, TINY.R) as L:
        x = ctypes.c_int64()
        assert lib.tide_layout_param(L.handle, 3, ctypes.byref(x), None, None, None) == tb.TIDE_ERR_INVALID
        assert lib.tide_layout_param(L.handle, -1, None, None, None, None) == tb.TIDE_ERR_INVALID
        assert lib.tide_layout_segment(L.handle, 0, 4, None, None, None, None) == tb.TIDE_ERR_INVALID
        buf = (ctypes.c_int64 * 6)()
        assert lib.tide_layout_copy_rs_items(L.handle, L.num_rs_chunks, 1, buf) == tb.TIDE_ERR_INVALID


def _fake_rs_args(L, C, base=1 << 32, g_step=1 << 20, s_step=1 << 20):
    grads = [base + (c * L.P + p) * g_step for c in range(C) for p in range(L.P)]
    shards = [base + (1 << 30) + r * s_step for r in range(L.R)]
    return grads, shards


def test_rs_rejects_bad_arguments_before_any_hip_call():
    lib = tb.load_library()
    with tide.Layout(TINY.shapes, TINY.R) as L:
        g, s = _fake_rs_args(L, 4)
        call = lambda gg, ss, C=4, form=0, count=0: lib.tide_rs_bf16_to_fp32(L.handle, C, _vp_array(gg), _vp_array(ss),
                                                                            form, count, None)
        INV = tb.TIDE_ERR_INVALID
        assert lib.tide_rs_bf16_to_fp32(None, 4, _vp_array(g), _vp_array(s), 0, 0, None) == INV
        assert lib.tide_rs_bf16_to_fp32(L.handle, 4, None, _vp_array(s), 0, 0, None) == INV
        assert call(g, s, C=0) == INV
        assert call(g, s, form=4) == INV                      # no such launch form
        assert call(g, s, form=tb.TIDE_LAUNCH_DEFAULT, count=1) == INV
        assert call(g, s, form=tb.TIDE_LAUNCH_CU_EXCLUSIVE, count=32) == INV   # at most 16 items
        assert call(g, s, C=5, form=tb.TIDE_LAUNCH_CU_EXCLUSIVE, count=16) == INV   # 2 items per group need C <= 4
        assert call(g, s, form=tb.TIDE_LAUNCH_PER_CU_CAP, count=65) == INV
        g2 = list(g); g2[5] = None
        assert call(g2, s) == INV                     # null gradient of a non-empty parameter
        g3 = list(g); g3[1] += 1
        assert call(g3, s) == INV                     # odd address for bf16
        s2 = list(s); s2[2] += 2
        assert call(g, s2) == INV                     # fp32 shard not 4-byte aligned
        s3 = list(s); s3[1] = s3[0] + 8
        assert call(g, s3) == INV                     # shards overlap
        s4 = list(s); s4[3] = g[2] + 4
        assert call(g, s4) == INV                     # shard overlaps a gradient
        assert lib.tide_last_hip_error() == 0


def test_ag_rejects_bad_arguments_before_any_hip_call():
    lib = tb.load_library()
    with tide.Layout(TINY.shapes, TINY.R) as L:
        stage = 1 << 32
        params = [(1 << 33) + p * (1 << 20) for p in range(L.P)]
        call = lambda st_, pp, mode=0, form=0, count=0: lib.tide_ag_place(L.handle, st_, _vp_array(pp), mode, form, count,
                                                                           None)
        INV = tb.TIDE_ERR_INVALID
        assert call(stage, params, mode=3) == INV
        assert call(stage, params, mode=-1) == INV
        assert call(stage, params, form=tb.TIDE_LAUNCH_PER_CU_CAP, count=2) == INV   # RS only
        assert call(stage, params, mode=tb.TIDE_AG_SDMA, form=tb.TIDE_LAUNCH_BOUNDED, count=8) == INV
        assert call(None, params) == INV
        assert call(stage + 1, params) == INV
        pp = list(params); pp[0] = None
        assert call(stage, pp) == INV
        pp = list(params); pp[1] = stage + 10
        assert call(stage, pp) == INV                 # parameter inside the stage
        pp = list(params); pp[2] = pp[0] + 2
        assert call(stage, pp) == INV                 # parameters overlap
        assert lib.tide_ag_place(None, stage, _vp_array(params), 0, 0, 0, None) == INV


def test_slot_entry_points_reject_bad_arguments_before_any_hip_call():
    lib = tb.load_library()
    INV = tb.TIDE_ERR_INVALID
    with tide.Layout(TINY.shapes, TINY.R) as L:
        slot = 1 << 32
        grads = [(1 << 33) + p * (1 << 20) for p in range(L.P)]
        pack = lambda gg, sl, form=0, count=0: lib.tide_slot_pack(L.handle, _vp_array(gg), sl, form, count, None)
        assert lib.tide_slot_pack(None, _vp_array(grads), slot, 0, 0, None) == INV
        assert lib.tide_slot_pack(L.handle, None, slot, 0, 0, None) == INV
        assert pack(grads, None) == INV
        assert pack(grads, slot + 1) == INV
        assert pack(grads, slot, form=tb.TIDE_LAUNCH_CU_EXCLUSIVE, count=9) == INV
        gg = list(grads); gg[1] = slot + 64
        assert pack(gg, slot) == INV                  # gradient inside the slot
        gg = list(grads); gg[0] = None
        assert pack(gg, slot) == INV
        slots = [(1 << 34) + c * (1 << 20) for c in range(4)]
        shards = [(1 << 35) + r * (1 << 20) for r in range(L.R)]
        rs = lambda sl, sh, C=4, form=0, count=0: lib.tide_rs_slots_bf16_to_fp32(L.handle, C, _vp_array(sl),
                                                                                 _vp_array(sh), form, count, None)
        assert rs(slots, shards, C=0) == INV
        assert rs(slots, shards, form=tb.TIDE_LAUNCH_BOUNDED, count=0) == INV
        ss = list(slots); ss[2] = None
        assert rs(ss, shards) == INV
        sh = list(shards); sh[0] = slots[1] + 8
        assert rs(slots, sh) == INV                   # shard overlaps a slot
        sh = list(shards); sh[1] += 2
        assert rs(slots, sh) == INV                   # misaligned fp32 shard
        assert lib.tide_last_hip_error() == 0


def test_probe_library_exports_and_rejects_bad_arguments():
    from all_gather_placement_amd import probe as pr

    lib = pr.load_probe_library()
    text = open(os.path.join(ROOT, "include", "tide_probe.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = sorted(set(re.findall(r"\b(tide_probe_[a-z0-9_]+)\s*\(", text)))
    assert names == ["tide_probe_build_id", "tide_probe_clock", "tide_probe_dma_rect_copies", "tide_probe_launch",
                     "tide_probe_mix", "tide_probe_stream_create_cu_mask", "tide_probe_stream_destroy",
                     "tide_probe_wall_clock_khz"]
    for n in names:
        assert hasattr(lib, n)
    assert lib.tide_probe_launch(0, 0, 10, None, None) == -1
    assert lib.tide_probe_launch(4, 7, 10, None, None) == -1
    assert lib.tide_probe_launch(4, 0, -1, None, None) == -1
    assert lib.tide_probe_clock(-1, 1 << 40, None) == -1
    assert lib.tide_probe_clock(10, None, None) == -1
    fake = 1 << 40
    assert lib.tide_probe_mix(3, 0, fake, fake, 8, 0, None) == -1           # C not 1, 2, 4 or 8
    assert lib.tide_probe_mix(8, 3, fake, fake, 8, 0, None) == -1           # bad mode
    assert lib.tide_probe_mix(8, 0, fake, fake, 0, 0, None) == -1           # no items
    assert lib.tide_probe_mix(8, 0, fake, fake, 1 << 31, 0, None) == -1     # grid too large
    assert lib.tide_probe_mix(8, 0, fake, None, 8, 0, None) == -1           # no destination
    assert lib.tide_probe_mix(8, 1, None, fake, 8, 0, None) == -1           # loads without sources
    assert lib.tide_probe_mix(8, 0, fake, fake, 8, -1, None) == -1          # negative local memory
    h = ctypes.c_void_p()
    assert lib.tide_probe_stream_create_cu_mask(0, 0, ctypes.byref(h)) == -1   # no CUs
    assert lib.tide_probe_stream_create_cu_mask(-1, 4, ctypes.byref(h)) == -1  # negative first CU
    assert lib.tide_probe_stream_create_cu_mask(0, 4, None) == -1              # nowhere to put the stream
    assert lib.tide_probe_stream_destroy(None) == -1
    assert h.value is None
    assert pr.clock_mhz([0, 100000, 5, 5 + 2_400_000], 100000) == 2400.0  # 1 ms of wall clock, 2.4M cycles
    # rectangular DMA copies: argument checks come before any HSA or HIP call
    a, b = 1 << 40, 1 << 41
    bad_rects = [(a, b, 64, 64, 0, 1), (a, b, 64, 64, 6, 1), (a, b, 64, 66, 8, 1), (a, b, 32, 64, 64, 1),
                 (a + 2, b, 64, 64, 8, 1), (None, b, 64, 64, 8, 1), (a, b, 64, 64, 8, 0), (a, b, 1 << 34, 1 << 34, 1 << 33, 1)]
    for r in bad_rects:
        arr = (pr.Rect * 1)(pr.Rect(*r))
        assert lib.tide_probe_dma_rect_copies(1, arr, 100, None) == -1, r
    assert lib.tide_probe_dma_rect_copies(0, (pr.Rect * 1)(), 100, None) == -1
    assert lib.tide_probe_dma_rect_copies(1, None, 100, None) == -1


def test_binding_checks_pointer_array_lengths_before_the_call():
    """The C entry points read host arrays of C*P, P and R pointers; the binding refuses Python
    sequences of other lengths instead of letting the library read past them (no HIP call made)."""
    lib = tb.load_library()
    with tide.Layout(TINY.shapes, TINY.R) as L:
        P, R = len(TINY.shapes), TINY.R
        base = 1 << 40
        grads = [[base + (c * P + p) * 4096 for p in range(P)] for c in range(2)]
        shards = [base + (1 << 30) + r * 4096 for r in range(R)]
        cases = [
            lambda: tb.tide_rs_bf16_to_fp32(L.handle, [grads[0][:-1], grads[1]], shards),
            lambda: tb.tide_rs_bf16_to_fp32(L.handle, grads, shards[:-1]),
            lambda: tb.tide_rs_bf16_to_fp32(L.handle, [], shards),
            lambda: tb.tide_ag_place(L.handle, base, grads[0][:-1]),
            lambda: tb.tide_slot_pack(L.handle, grads[0] + [base], base + (1 << 32)),
            lambda: tb.tide_rs_slots_bf16_to_fp32(L.handle, [base], shards + [base]),
            lambda: tb.tide_rs_prepare(L.handle, grads, shards[:1]),
            lambda: tb.tide_ag_prepare(L.handle, base, []),
            lambda: tb.tide_slot_pack_prepare(L.handle, grads[0][:1], base),
            lambda: tb.tide_rs_slots_prepare(L.handle, [base], []),
        ]
        for case in cases:
            with pytest.raises(tide.TideError, match="INVALID"):
                case()
        assert lib.tide_last_hip_error() == 0


def test_binding_rejects_tensors_on_mixed_devices():
    """Tensor arguments must all sit on one device (the current one when a GPU is present)."""
    import torch

    class FakeTensor:  # duck-typed like a torch tensor, on a chosen device; never dereferenced
        def __init__(self, dev):
            self.device = torch.device("cuda", dev)
            self.dtype = torch.bfloat16
            self.is_cuda = True

        def data_ptr(self):
            return 1 << 40

    with tide.Layout(TINY.shapes, TINY.R) as L:
        grads = [[FakeTensor(0) for _ in range(L.P)] for _ in range(2)]
        shards = [FakeTensor(0) for _ in range(L.R - 1)] + [FakeTensor(1)]
        with pytest.raises(ValueError, match="current device"):
            L.rs_bf16_to_fp32(grads, shards)
        with pytest.raises(ValueError, match="current device"):
            L.ag_place(FakeTensor(1), [FakeTensor(0) for _ in range(L.P)])


def test_launch_forms_match_the_header():
    """The launch-form enum and limits in include/tide.h and the binding's Launch agree."""
    text = open(os.path.join(ROOT, "include", "tide.h")).read()
    for name in ("TIDE_LAUNCH_DEFAULT", "TIDE_LAUNCH_BOUNDED", "TIDE_LAUNCH_CU_EXCLUSIVE", "TIDE_LAUNCH_PER_CU_CAP"):
        value = int(re.search(name + r" = (\d+)", text).group(1))
        assert getattr(tide, name) == value, name
    for name in ("TIDE_MAX_WGS_PER_CU", "TIDE_CU_EXCLUSIVE_MAX_ITEMS", "TIDE_NOALLOC_MAX_PTRS"):
        assert getattr(tide, name) == int(re.search(r"#define " + name + r" (\d+)", text).group(1)), name
    assert tide.Launch() == tide.Launch.default() == (tide.TIDE_LAUNCH_DEFAULT, 0)
    assert tide.Launch.bounded(512) == (tide.TIDE_LAUNCH_BOUNDED, 512)
    assert tide.Launch.cu_exclusive(16) == (tide.TIDE_LAUNCH_CU_EXCLUSIVE, 16)
    assert tide.Launch.per_cu_cap(6) == (tide.TIDE_LAUNCH_PER_CU_CAP, 6)
    assert str(tide.Launch.bounded(3)) == "bounded(3)" and str(tide.Launch()) == "default"
    for bad in (lambda: tide.Launch.bounded(0), lambda: tide.Launch.cu_exclusive(9), lambda: tide.Launch.cu_exclusive(0),
                lambda: tide.Launch.cu_exclusive(32),
                lambda: tide.Launch.per_cu_cap(tide.TIDE_MAX_WGS_PER_CU + 1)):
        with pytest.raises(ValueError):
            bad()


def test_build_id_matches_the_sources():
    """Each library carries the build id of the sources in the tree it was built from."""
    from all_gather_placement_amd import build

    for lib in (build.LIB, build.PROBE_LIB):
        assert build.built_id(lib) == build.source_hash(lib)
        assert len(build.source_hash(lib)) == 16
    assert tb.load_library().tide_build_id().decode() == build.source_hash(build.LIB)


def test_library_built_from_other_sources_is_refused_or_rebuilt(monkeypatch):
    """A library whose build id differs from the sources beside it is refused by the binding, and
    ensure_built() rebuilds it.  The mismatch is faked by changing the id the sources are expected to
    have; no file is edited."""
    import ctypes

    from all_gather_placement_amd import build, probe, tide

    lib = ctypes.CDLL(build.LIB)
    build.check_current(build.LIB, loaded=lib)  # the real one passes
    monkeypatch.setattr(build, "source_hash", lambda lib=build.LIB, extra=(): "0123456789abcdef")
    with pytest.raises(RuntimeError, match="other sources"):
        build.check_current(build.LIB, loaded=lib)
    with pytest.raises(RuntimeError, match="other sources"):
        tide.load_library(tide.library_path())  # an explicit load re-checks
    monkeypatch.setattr(probe, "_lib", None)
    with pytest.raises(RuntimeError, match="other sources"):
        probe.load_probe_library()
    monkeypatch.setattr(probe, "_lib", None)
    assert not build.is_current(build.LIB) and not build.is_current(build.PROBE_LIB)
    rebuilt = []
    monkeypatch.setattr(build, "build", lambda verbose=False: rebuilt.append(True) or build.LIB)
    build.ensure_built()
    assert rebuilt == [True]
