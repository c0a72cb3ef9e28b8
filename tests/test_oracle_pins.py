"""Pins of the CPU oracle against things other than itself (CPU only).

Every check here is independent of the oracle's own code path: hand-worked golden values,
torch's own bf16 conversion and dim-0 chunking (FSDP2 shards dim 0 with torch.chunk), exact
integer arithmetic, math.fsum, brute-force loops, and IEEE cases derived by hand.  The mutant
tests at the end plant plausible mistakes in copies of the oracle and check that at least one pin
catches each of them.
"""
import math
import os

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

import oracle
from oracle import geometry as ogeo
from oracle import rs as ors
from oracle import ag as oag
from tests.conftest import golden_path
from workloads import TINY, CONFIGS, ORDERED, group_grads_np, normal_bf16_bits, f32_to_bf16_bits

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


# ---------------------------------------------------------------------------------------------
# Geometry
# ---------------------------------------------------------------------------------------------

def _read_geometry_golden():
    rows = {}
    for line in open(golden_path("tiny_geometry.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        parts = line.split()
        rows[parts[0]] = [int(x) for x in parts[1:]]
    return rows


def test_tiny_geometry_matches_hand_worked_values():
    gold = _read_geometry_golden()
    geo, S = ogeo.group_geometry(TINY.shapes, TINY.R)
    assert S == gold["S"][0]
    pad = 0
    for name, g in zip(TINY.names, geo):
        rows, L, m, e, o, *v = gold[name]
        assert (g.rows, g.L, g.m, g.e, g.o) == (rows, L, m, e, o)
        vv = [ogeo.valid_rows(g.rows, g.m, r) for r in range(TINY.R)]
        assert vv == v
        pad += sum((g.m - x) * g.L for x in vv)
    assert pad == gold["padding"][0]


def check_valid_rows_against_torch_chunk(valid_rows_fn, ceil_fn) -> bool:
    """FSDP2 shards dim 0 with torch.chunk; its per-rank row counts must equal v(p, r)."""
    for rows in range(0, 40):
        for R in range(1, 12):
            m = ceil_fn(rows, R)
            chunks = [int(t.numel()) for t in torch.chunk(torch.arange(rows), R)] if rows else []
            chunks += [0] * (R - len(chunks))
            if [valid_rows_fn(rows, m, r) for r in range(R)] != chunks:
                return False
            if chunks and max(chunks) != m:
                return False
    return True


def test_valid_rows_equal_torch_chunk():
    assert check_valid_rows_against_torch_chunk(ogeo.valid_rows, lambda a, b: -(-a // b))


@pytest.mark.parametrize("cfg", ORDERED, ids=lambda c: c.name)
def test_config_geometry_closed_forms(cfg):
    geo, S = ogeo.group_geometry(cfg.shapes, cfg.R)
    # prefix offsets partition [0, S)
    assert geo[0].o == 0
    for a, b in zip(geo, geo[1:]):
        assert b.o == a.o + a.e
    assert geo[-1].o + geo[-1].e == S
    # every row lands on exactly one rank
    for g in geo:
        assert sum(ogeo.valid_rows(g.rows, g.m, r) for r in range(cfg.R)) == g.rows
    if cfg.name != "tiny":
        # all large groups divide evenly: no padding, R*S == total numel
        assert cfg.R * S == cfg.numel()


def test_large_config_sizes():
    # S per config (elements): computed by hand from the shapes in the workload definitions.
    assert ogeo.group_geometry(CONFIGS["llama3_1_8b_layer"].shapes, 8)[1] == 27_264_000
    assert ogeo.group_geometry(CONFIGS["llama3_1_70b_layer"].shapes, 8)[1] == 106_956_800
    assert ogeo.group_geometry(CONFIGS["qwen3_30b_a3b"].shapes, 16)[1] == 38_945_024
    assert ogeo.group_geometry(CONFIGS["wan2_2_block"].shapes, 64)[1] == 5_489_520
    assert CONFIGS["qwen3_30b_a3b"].P == 391 and CONFIGS["wan2_2_block"].P == 21


def test_geometry_rejects_bad_shapes():
    with pytest.raises(ValueError):
        ogeo.group_geometry([()], 4)
    with pytest.raises(ValueError):
        ogeo.group_geometry([(3, -1)], 4)
    with pytest.raises(ValueError):
        ogeo.group_geometry([(3,)], 0)


# ---------------------------------------------------------------------------------------------
# widen and bf16 rounding (input side) against torch's own conversions
# ---------------------------------------------------------------------------------------------

def test_widen_matches_torch_bfloat16_conversion():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    got = ors.widen(bits)
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin].view(np.uint32), ref[fin].view(np.uint32))
    assert np.array_equal(np.isnan(got), np.isnan(ref))


def test_input_rounding_matches_torch():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(200_000).astype(np.float32) * np.float32(10.0) ** rng.integers(-30, 30, 200_000).astype(np.float32))
    x = x[np.isfinite(x)]
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(f32_to_bf16_bits(x), ref)


# ---------------------------------------------------------------------------------------------
# Reduce-scatter
# ---------------------------------------------------------------------------------------------

def _read_sum_cases():
    cases = []
    for line in open(golden_path("fp32_sum_cases.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        ins, out, _why = [s.strip() for s in line.split(";")]
        cases.append(([int(h, 16) for h in ins.split()], int(out, 16)))
    return cases


def check_sum_cases(rs_fn) -> bool:
    """Each golden case as a one-element group (shape (1,), R=1) with C contributors."""
    for ins, expect in _read_sum_cases():
        grads = [[np.array([b], dtype=np.uint16)] for b in ins]
        y = rs_fn(grads, [(1,)], 1)
        if int(np.asarray(y, dtype=np.float32).view(np.uint32).ravel()[0]) != expect:
            return False
    return True


def test_golden_fp32_sum_cases():
    assert check_sum_cases(ors.reduce_scatter)


def test_rs_sampled_matches_golden_cases():
    for ins, expect in _read_sum_cases():
        y = ors.rs_sampled(np.array(ins, dtype=np.uint16).reshape(-1, 1))
        assert int(y.view(np.uint32)[0]) == expect


def _tiny_grads(C=None):
    return group_grads_np(TINY, C)


def test_tiny_rs_equals_brute_force():
    g = _tiny_grads()
    Y = oracle.reduce_scatter(g, TINY.shapes, TINY.R)
    B = oracle.brute_reduce_scatter(g, TINY.shapes, TINY.R)
    assert np.array_equal(Y.view(np.uint32), B.view(np.uint32))


@st.composite
def tiny_groups(draw):
    R = draw(st.integers(1, 9))
    C = draw(st.integers(1, 5))
    P = draw(st.integers(1, 5))
    shapes = []
    for _ in range(P):
        nd = draw(st.integers(1, 3))
        rows = draw(st.integers(0, 13))
        rest = [draw(st.integers(1, 4)) for _ in range(nd - 1)]
        shapes.append(tuple([rows] + rest))
    seed = draw(st.integers(0, 2**31 - 1))
    return R, C, shapes, seed


def _rand_grads(C, shapes, seed, sigma=1.0):
    return [[normal_bf16_bits(s, sigma, 99, seed, c, p) for p, s in enumerate(shapes)] for c in range(C)]


@settings(max_examples=60, deadline=None)
@given(tiny_groups())
def test_hypothesis_rs_equals_brute_force(group):
    R, C, shapes, seed = group
    g = _rand_grads(C, shapes, seed)
    Y = oracle.reduce_scatter(g, shapes, R)
    B = oracle.brute_reduce_scatter(g, shapes, R)
    assert np.array_equal(Y.view(np.uint32), B.view(np.uint32))


def test_single_contributor_is_exact_widen_via_torch():
    g = _tiny_grads(1)
    Y = oracle.reduce_scatter(g, TINY.shapes, TINY.R)
    geo, S = ogeo.group_geometry(TINY.shapes, TINY.R)
    for p, gg in enumerate(geo):
        t = torch.from_numpy(g[0][p].astype(np.int16)).view(torch.bfloat16).float().reshape(gg.rows, gg.L)
        for r, piece in enumerate(torch.chunk(t, TINY.R, dim=0)):
            n = piece.numel()
            got = Y[r, gg.o: gg.o + n]
            assert np.array_equal(got.view(np.uint32), piece.reshape(-1).numpy().view(np.uint32))


def test_identical_contributors_sum_to_c_times_x():
    x = normal_bf16_bits((200, 7), 1.0, 7, 1)
    for C in (1, 2, 3, 5, 8, 16):
        Y = oracle.reduce_scatter([[x]] * C, [(200, 7)], 1)[0]
        expect = np.array([C * float(v) for v in ors.widen(x).ravel()], dtype=np.float64).astype(np.float32)
        assert np.array_equal(Y.view(np.uint32), expect.view(np.uint32))


def _integer_grads(C, shapes, seed, with_ints=False):
    """bf16 holding small integers |x| <= 16: every partial sum is exact in fp32."""
    rng = np.random.default_rng(seed)
    out, ints_out = [], []
    for c in range(C):
        row, irow = [], []
        for s in shapes:
            ints = rng.integers(-16, 17, size=s)
            row.append(f32_to_bf16_bits(ints.astype(np.float32)).reshape(s))
            irow.append(ints.astype(np.int64))
        out.append(row)
        ints_out.append(irow)
    return (out, ints_out) if with_ints else out


def check_integer_sums(rs_fn) -> bool:
    """Exact integer sums (Python ints) at every valid position; zeros at padding."""
    shapes = [(7, 5), (16, 3), (1, 9), (5,)]
    R, C = 4, 6
    g, ints = _integer_grads(C, shapes, 5, with_ints=True)
    Y = np.asarray(rs_fn(g, shapes, R))
    geo, S = ogeo.group_geometry(shapes, R)
    for p, gg in enumerate(geo):
        full = sum(ints[c][p] for c in range(C)).reshape(gg.rows * gg.L)
        for r in range(R):
            v = ogeo.valid_rows(gg.rows, gg.m, r)
            seg = Y[r, gg.o: gg.o + gg.e]
            if not np.array_equal(seg[: v * gg.L].astype(np.int64), full[r * gg.m * gg.L: (r * gg.m + v) * gg.L]):
                return False
            if np.any(seg[v * gg.L:].view(np.uint32) != 0):
                return False
    return True


def test_integer_inputs_exact_and_permutation_invariant():
    assert check_integer_sums(oracle.reduce_scatter)
    shapes = [(7, 5), (16, 3)]
    g = _integer_grads(5, shapes, 11)
    Y0 = oracle.reduce_scatter(g, shapes, 3)
    for perm in ([4, 3, 2, 1, 0], [2, 0, 4, 1, 3]):
        Yp = oracle.reduce_scatter([g[i] for i in perm], shapes, 3)
        assert np.array_equal(Y0, Yp)


def test_all_negative_zero_stays_negative_zero():
    z = np.full((6, 4), 0x8000, dtype=np.uint16)
    Y = oracle.reduce_scatter([[z]] * 4, [(6, 4)], 4)
    geo, S = ogeo.group_geometry([(6, 4)], 4)
    # rows 0..5 over m=2: ranks 0,1,2 full, rank 3 padding only
    bits = Y.view(np.uint32)
    assert np.all(bits[:3] == 0x80000000)
    assert np.all(bits[3] == 0)  # padding is +0.0


def test_r1_is_concatenation_of_full_sums():
    g = _tiny_grads()
    Y = oracle.reduce_scatter(g, TINY.shapes, 1)
    parts = []
    for p in range(TINY.P):
        acc = ors.widen(g[0][p]).ravel().copy()
        for c in range(1, TINY.C):
            acc = acc + ors.widen(g[c][p]).ravel()
        parts.append(acc)
    assert np.array_equal(Y[0].view(np.uint32), np.concatenate(parts).view(np.uint32))


def test_concatenated_unpadded_shards_equal_full_sum_llama_norms():
    # The two norm parameters of the Llama-8B group, R=8: shards concatenated per parameter and
    # unpadded give the full-tensor sum (a property stated for the method's output).
    shapes = [(4096,), (4096,), (12, 5)]
    g = _rand_grads(8, shapes, 4, sigma=1e-3)
    Y = oracle.reduce_scatter(g, shapes, 8)
    geo, S = ogeo.group_geometry(shapes, 8)
    for p, gg in enumerate(geo):
        cat = np.concatenate([Y[r, gg.o: gg.o + gg.e] for r in range(8)])[: gg.rows * gg.L]
        acc = ors.widen(g[0][p]).ravel()
        for c in range(1, 8):
            acc = acc + ors.widen(g[c][p]).ravel()
        assert np.array_equal(cat.view(np.uint32), acc.view(np.uint32))


def test_error_bound_against_exact_sum():
    shapes = [(64, 33)]
    C = 8
    g = _rand_grads(C, shapes, 21, sigma=1e-3)
    Y = oracle.reduce_scatter(g, shapes, 1)[0]
    W = np.stack([ors.widen(g[c][0]).ravel().astype(np.float64) for c in range(C)])
    for j in range(W.shape[1]):
        exact = math.fsum(W[:, j])
        bound = (C - 1) * 2.0 ** -24 * float(np.sum(np.abs(W[:, j])))
        assert abs(float(Y[j]) - exact) <= bound


def test_rs_sampled_and_locate_match_full_rs():
    g = _tiny_grads()
    Y = oracle.reduce_scatter(g, TINY.shapes, TINY.R)
    geo, S = ogeo.group_geometry(TINY.shapes, TINY.R)
    for r in range(TINY.R):
        for k in range(S):
            p, src = ors.locate(TINY.shapes, TINY.R, r, k)
            if src is None:
                assert Y[r, k].view(np.uint32) == 0
                continue
            vals = np.array([g[c][p].ravel()[src] for c in range(TINY.C)], dtype=np.uint16).reshape(-1, 1)
            assert ors.rs_sampled(vals).view(np.uint32)[0] == Y[r, k].view(np.uint32)


# ---------------------------------------------------------------------------------------------
# All-gather placement
# ---------------------------------------------------------------------------------------------

def check_ag_against_torch_chunks(ag_fn, shapes, R, stage) -> bool:
    """FSDP2-style copy-out with torch: rank r's piece of p is stage_r[o_p : o_p + numel(chunk r)]."""
    geo, S = ogeo.group_geometry(shapes, R)
    st_t = torch.from_numpy(stage.astype(np.int16)).reshape(R, S)
    got = ag_fn(stage, shapes, R)
    for p, (gg, shape) in enumerate(zip(geo, shapes)):
        sizes = [int(t.numel()) for t in torch.chunk(torch.empty(gg.rows, gg.L), R, dim=0)] if gg.rows else []
        sizes += [0] * (R - len(sizes))
        pieces = [st_t[r, gg.o: gg.o + sizes[r]] for r in range(R)]
        ref = torch.cat(pieces).numpy().view(np.uint16).reshape(shape)
        if not np.array_equal(np.asarray(got[p]).reshape(shape), ref):
            return False
    return True


def test_tiny_ag_against_brute_and_torch():
    geo, S = ogeo.group_geometry(TINY.shapes, TINY.R)
    stage = normal_bf16_bits((TINY.R * S,), 1.0, 0, 77)
    A = oracle.all_gather_place(stage, TINY.shapes, TINY.R)
    B = oracle.brute_all_gather_place(stage, TINY.shapes, TINY.R)
    for a, b in zip(A, B):
        assert np.array_equal(a, b)
    assert check_ag_against_torch_chunks(oracle.all_gather_place, TINY.shapes, TINY.R, stage)


@settings(max_examples=60, deadline=None)
@given(tiny_groups())
def test_hypothesis_ag_against_brute_and_torch(group):
    R, _C, shapes, seed = group
    geo, S = ogeo.group_geometry(shapes, R)
    stage = normal_bf16_bits((R * S,), 1.0, 98, seed)
    A = oracle.all_gather_place(stage, shapes, R)
    B = oracle.brute_all_gather_place(stage, shapes, R)
    for a, b in zip(A, B):
        assert np.array_equal(a, b)
    assert check_ag_against_torch_chunks(oracle.all_gather_place, shapes, R, stage)


def test_ag_never_reads_stage_padding():
    geo, S = ogeo.group_geometry(TINY.shapes, TINY.R)
    stage = normal_bf16_bits((TINY.R * S,), 1.0, 0, 78).reshape(TINY.R, S)
    POISON = 0x7FC1  # a quiet-NaN bf16 pattern that normal draws never produce
    for gg in geo:
        for r in range(TINY.R):
            v = ogeo.valid_rows(gg.rows, gg.m, r)
            stage[r, gg.o + v * gg.L: gg.o + gg.e] = POISON
    params = oracle.all_gather_place(stage.ravel(), TINY.shapes, TINY.R)
    assert not any(np.any(p == POISON) for p in params)
    assert sum(p.size for p in params) == TINY.numel()


def test_ag_then_single_contributor_rs_round_trips():
    geo, S = ogeo.group_geometry(TINY.shapes, TINY.R)
    stage = normal_bf16_bits((TINY.R * S,), 1.0, 0, 79)
    params = oracle.all_gather_place(stage, TINY.shapes, TINY.R)
    Y = oracle.reduce_scatter([params], TINY.shapes, TINY.R)
    W = ors.widen(stage).reshape(TINY.R, S)
    for gg in geo:
        for r in range(TINY.R):
            v = ogeo.valid_rows(gg.rows, gg.m, r)
            a, b, e = gg.o, gg.o + v * gg.L, gg.o + gg.e
            assert np.array_equal(Y[r, a:b].view(np.uint32), W[r, a:b].view(np.uint32))
            assert np.all(Y[r, b:e].view(np.uint32) == 0)


def test_ag_copies_nan_bits_exactly():
    shapes = [(3, 2)]
    stage = np.array([0x7FC0, 0xFFC1, 0x7F81, 0x0001, 0x8000, 0x7F80], dtype=np.uint16)
    (p,) = oracle.all_gather_place(stage, shapes, 1)
    assert np.array_equal(p.ravel(), stage)


# ---------------------------------------------------------------------------------------------
# Planted mistakes: each mutant of the oracle must fail at least one of the pins above.
# ---------------------------------------------------------------------------------------------

def _rs_reversed(grads, shapes, R):
    Y = ors.pack_contributor(grads[-1], shapes, R)
    for c in range(len(grads) - 2, -1, -1):
        Y = Y + ors.pack_contributor(grads[c], shapes, R)
    return Y


def _rs_from_zero(grads, shapes, R):
    Y = np.zeros_like(ors.pack_contributor(grads[0], shapes, R))
    for c in range(len(grads)):
        Y = Y + ors.pack_contributor(grads[c], shapes, R)
    return Y


def _rs_dropped_last(grads, shapes, R):
    return ors.reduce_scatter(grads[:-1] if len(grads) > 1 else grads, shapes, R)


def _rs_offset_by_one(grads, shapes, R):
    Y = ors.reduce_scatter(grads, shapes, R)
    return np.roll(Y, 1, axis=1)


def _ag_transposed(stage, shapes, R):
    geo, S = ogeo.group_geometry(shapes, R)
    st_ = np.asarray(stage, dtype=np.uint16).reshape(S, R).T  # wrong: slot-major read
    out = []
    for g, shape in zip(geo, shapes):
        out.append(st_[:, g.o: g.o + g.e].reshape(R * g.m, g.L)[: g.rows].reshape(shape))
    return out


def test_mutants_are_caught():
    assert not check_sum_cases(_rs_reversed)
    assert not check_sum_cases(_rs_from_zero)
    assert not check_integer_sums(_rs_dropped_last)
    assert not check_integer_sums(_rs_offset_by_one)
    assert not check_valid_rows_against_torch_chunk(ogeo.valid_rows, lambda a, b: a // b)  # floor for ceil
    geo, S = ogeo.group_geometry(TINY.shapes, TINY.R)
    stage = normal_bf16_bits((TINY.R * S,), 1.0, 0, 80)
    assert not check_ag_against_torch_chunks(_ag_transposed, TINY.shapes, TINY.R, stage)


# ---------------------------------------------------------------------------------------------
# Slot-Reuse staging (pack into an all-gather slot that is free again, then reduce from the slots)
# ---------------------------------------------------------------------------------------------

@settings(max_examples=40, deadline=None)
@given(tiny_groups())
def test_slot_pack_is_inverse_of_ag_and_rs_from_slots_equals_in_place(group):
    R, C, shapes, seed = group
    g = _rand_grads(C, shapes, seed)
    geo, S = ogeo.group_geometry(shapes, R)
    slots = [oracle.pack_slot(g[c], shapes, R) for c in range(C)]
    for c in range(C):
        # placing a packed slot gives the gradients back, bit for bit
        back = oracle.all_gather_place(slots[c], shapes, R)
        for a, b in zip(back, g[c]):
            assert np.array_equal(a, b)
        # the bf16 slot widened is the stock fp32 pack
        assert np.array_equal(ors.widen(slots[c]).reshape(R, S).view(np.uint32),
                              ors.pack_contributor(g[c], shapes, R).view(np.uint32))
    Y = oracle.rs_from_slots(slots, shapes, R)
    assert np.array_equal(Y.view(np.uint32), oracle.reduce_scatter(g, shapes, R).view(np.uint32))
    assert np.array_equal(Y.view(np.uint32), oracle.brute_reduce_scatter(g, shapes, R).view(np.uint32))


def test_rs_from_slots_ignores_slot_padding():
    geo, S = ogeo.group_geometry(TINY.shapes, TINY.R)
    g = _tiny_grads()
    slots = [oracle.pack_slot(g[c], TINY.shapes, TINY.R).reshape(TINY.R, S) for c in range(TINY.C)]
    for s in slots:  # garbage in the padding of every slot
        for gg in geo:
            for r in range(TINY.R):
                v = ogeo.valid_rows(gg.rows, gg.m, r)
                s[r, gg.o + v * gg.L: gg.o + gg.e] = 0x7FC1
    Y = oracle.rs_from_slots([s.ravel() for s in slots], TINY.shapes, TINY.R)
    assert np.array_equal(Y.view(np.uint32), oracle.reduce_scatter(g, TINY.shapes, TINY.R).view(np.uint32))
