"""GPU parity of the HIP reduce-scatter and all-gather placement against the CPU oracle.

Every group, from the tiny one to the four full-size layer groups, is compared element by element
(bit-exact) with the oracle on the same seeded inputs; the full-size groups are reduced by the oracle
one run of parameters at a time, from contributor bytes read back from the device.  Properties that
hold at any size are checked beside it (bit-exact agreement with a plain torch fixed-order fp32 sum,
padding zeros, write-once coverage, the AG->RS round trip).
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import geometry as ogeo
from oracle import rs as ors
from all_gather_placement_amd import (Layout, TIDE_AG_COPY2D, TIDE_AG_KERNEL, TIDE_AG_SDMA, TideError,
                                      Launch)
from workloads import ORDERED, TINY, normal_bf16_bits, normal_bf16_cuda, f32_to_bf16_bits

pytestmark = pytest.mark.gpu

POISON_F32 = 0x7FC0DEAD  # a NaN pattern no sum produces from these inputs
POISON_BF16 = 0x7FC1


def say(msg):
    print(f"[gpu-parity] {msg}", flush=True)


def dev_bf16(bits: np.ndarray, pad_elems: int = 0):
    """Upload uint16 bits as a contiguous bf16 cuda tensor; pad_elems shifts it off 16-B alignment."""
    flat = np.ascontiguousarray(bits, dtype=np.uint16).ravel()
    if pad_elems == 0:
        return torch.from_numpy(flat.view(np.int16).copy()).cuda().view(torch.bfloat16).reshape(bits.shape)
    buf = torch.empty(flat.size + pad_elems + 8, dtype=torch.int16, device="cuda")
    view = buf[pad_elems: pad_elems + flat.size]
    view.copy_(torch.from_numpy(flat.view(np.int16).copy()))
    return view.view(torch.bfloat16).reshape(bits.shape)


def host_bits_bf16(t) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host_bits_f32(t) -> np.ndarray:
    return t.detach().contiguous().view(torch.int32).cpu().numpy().view(np.uint32)


def poisoned_shards(R, S, pad_elems=0):
    out = []
    for r in range(R):
        buf = torch.full((S + pad_elems + 4,), POISON_F32, dtype=torch.int32, device="cuda")
        out.append(buf[pad_elems: pad_elems + S].view(torch.float32))
    return out


def run_rs(shapes, R, grads_bits, launch=Launch(), g_pad=None, s_pad=0, stream=None):
    """Upload, run the HIP RS, return (R, S) uint32 bits."""
    C = len(grads_bits)
    g_pad = g_pad or (lambda c, p: 0)
    grads = [[dev_bf16(grads_bits[c][p], g_pad(c, p)) for p in range(len(shapes))] for c in range(C)]
    with Layout(shapes, R) as L:
        shards = poisoned_shards(R, L.S, s_pad)
        L.rs_bf16_to_fp32(grads, shards, launch=launch, stream=stream)
        torch.cuda.synchronize()
        return np.stack([host_bits_f32(s) for s in shards]) if L.S else np.zeros((R, 0), np.uint32)


def assert_rs_equal(got_bits, want_f32):
    want = np.asarray(want_f32, dtype=np.float32).view(np.uint32)
    assert got_bits.shape == want.shape
    bad = np.nonzero(got_bits != want)
    if bad[0].size:
        i = tuple(b[0] for b in bad)
        raise AssertionError(f"{bad[0].size} mismatches; first at {i}: got {got_bits[i]:#010x} want {want[i]:#010x}")


def run_ag(shapes, R, stage_bits, mode=TIDE_AG_KERNEL, launch=Launch(), st_pad=0, p_pad=None):
    p_pad = p_pad or (lambda p: 0)
    stage = dev_bf16(stage_bits, st_pad)
    params = []
    for p, s in enumerate(shapes):
        n = int(np.prod(s, dtype=np.int64))
        buf = torch.full((n + p_pad(p) + 8,), POISON_BF16, dtype=torch.int16, device="cuda")
        params.append(buf[p_pad(p): p_pad(p) + n].view(torch.bfloat16).reshape(s))
    with Layout(shapes, R) as L:
        L.ag_place(stage, params, mode=mode, launch=launch)
        torch.cuda.synchronize()
    return [host_bits_bf16(q) for q in params]


# ------------------------------------------------------------------------------------------------
# Small groups: full element-by-element parity
# ------------------------------------------------------------------------------------------------

def test_tiny_rs_bit_exact(gpu_available):
    say("tiny RS")
    g = [[normal_bf16_bits(s, TINY.sigma, TINY.cfg_id, c, p) for p, s in enumerate(TINY.shapes)] for c in range(TINY.C)]
    want = oracle.reduce_scatter(g, TINY.shapes, TINY.R)
    for launch in (Launch.default(), Launch.bounded(1), Launch.bounded(2), Launch.bounded(5), Launch.per_cu_cap(3),
                   Launch.cu_exclusive(1), Launch.cu_exclusive(8), Launch.cu_exclusive(16)):
        assert_rs_equal(run_rs(TINY.shapes, TINY.R, g, launch=launch), want)


@pytest.mark.parametrize("mode", [TIDE_AG_KERNEL, TIDE_AG_SDMA, TIDE_AG_COPY2D], ids=["kernel", "sdma", "copy2d"])
def test_tiny_ag_bit_exact(gpu_available, mode):
    say(f"tiny AG mode={mode}")
    geo, S = ogeo.group_geometry(TINY.shapes, TINY.R)
    stage = normal_bf16_bits((TINY.R * S,), 1.0, TINY.cfg_id, 1 << 20, 0)
    # poison the stage padding: it must never reach a parameter
    st2 = stage.reshape(TINY.R, S).copy()
    for gg in geo:
        for r in range(TINY.R):
            v = ogeo.valid_rows(gg.rows, gg.m, r)
            st2[r, gg.o + v * gg.L: gg.o + gg.e] = POISON_BF16
    stage = st2.ravel()
    want = oracle.all_gather_place(stage, TINY.shapes, TINY.R)
    got = run_ag(TINY.shapes, TINY.R, stage, mode=mode)
    for a, b in zip(got, want):
        assert np.array_equal(a, b)


GROUPS = [
    # (shapes, R, C): ragged tails, rows < R, empty parameters, 1-D/3-D; C <= 16 runs kernels compiled
    # for that C (16 the largest), C > 16 the runtime-C kernels
    ([(7, 5), (16, 3), (1, 9)], 4, 4),
    ([(1000, 37), (4099,), (333, 65), (0, 4), (3, 2, 5)], 8, 8),
    ([(5, 1), (2,), (9, 3, 3)], 9, 3),
    ([(20000,), (129, 257)], 3, 1),
    ([(64, 64)], 1, 2),
    ([(77, 31), (3,)], 16, 10),
    ([(40000, 3), (11, 4097)], 5, 5),
    ([(2, 3)], 7, 12),
    ([(300, 70), (17,), (2048, 3)], 4, 16),
    ([(129, 33), (5000,), (0, 3)], 6, 18),
    ([(33, 9), (70001,)], 3, 40),
]


@pytest.mark.parametrize("case", range(len(GROUPS)))
def test_groups_rs_bit_exact(gpu_available, case):
    shapes, R, C = GROUPS[case]
    say(f"group {case}: shapes={shapes} R={R} C={C}")
    g = [[normal_bf16_bits(s, 1.0, 50 + case, c, p) for p, s in enumerate(shapes)] for c in range(C)]
    want = oracle.reduce_scatter(g, shapes, R)
    # every launch form: the default (CU-exclusive, shaped for C), short bounded launches, single-item
    # workgroups under a per-CU cap, and CU-exclusive workgroups of one item per group and, where C
    # allows it, of several items per group
    forms = [Launch.default(), Launch.bounded(3), Launch.per_cu_cap(2), Launch.cu_exclusive(3)]
    forms += [Launch.cu_exclusive(16)] if C <= 4 else []
    for launch in forms:
        assert_rs_equal(run_rs(shapes, R, g, launch=launch), want)


@pytest.mark.parametrize("case", range(len(GROUPS)))
@pytest.mark.parametrize("mode", [TIDE_AG_KERNEL, TIDE_AG_SDMA, TIDE_AG_COPY2D], ids=["kernel", "sdma", "copy2d"])
def test_groups_ag_bit_exact(gpu_available, case, mode):
    shapes, R, _ = GROUPS[case]
    say(f"group {case} AG mode={mode}")
    geo, S = ogeo.group_geometry(shapes, R)
    stage = normal_bf16_bits((R * S,), 1.0, 60 + case, 0)
    want = oracle.all_gather_place(stage, shapes, R)
    forms = (Launch.default(), Launch.bounded(1), Launch.bounded(3), Launch.bounded(1024), Launch.cu_exclusive(5))
    for launch in (forms if mode == TIDE_AG_KERNEL else (Launch.default(),)):
        got = run_ag(shapes, R, stage, mode=mode, launch=launch)
        for a, b in zip(got, want):
            assert np.array_equal(a, b), launch


@pytest.mark.parametrize("g_off", [0, 1, 3, 7])
@pytest.mark.parametrize("s_off", [0, 1, 2])
@pytest.mark.parametrize("C", [6, 20])
def test_rs_alignment_sweep(gpu_available, g_off, s_off, C):
    """Base pointers shifted off 16-byte alignment: the element path must agree bit for bit, for a
    compiled contributor count and for the runtime-C kernel."""
    shapes, R = [(300, 17), (1025,), (8, 64)], 4
    say(f"alignment g_off={g_off} s_off={s_off} C={C}")
    g = [[normal_bf16_bits(s, 1.0, 70, c, p) for p, s in enumerate(shapes)] for c in range(C)]
    want = oracle.reduce_scatter(g, shapes, R)
    # mixed offsets across contributors when g_off > 0; one launch, and short bounded launches
    for launch in (Launch.default(), Launch.bounded(2), Launch.per_cu_cap(6)):
        got = run_rs(shapes, R, g, launch=launch, g_pad=lambda c, p: (g_off * (c + 1)) % 8, s_pad=s_off)
        assert_rs_equal(got, want)


@pytest.mark.parametrize("st_off,p_off", [(0, 0), (1, 0), (0, 3), (5, 5), (2, 6)])
def test_ag_alignment_sweep(gpu_available, st_off, p_off):
    shapes, R = [(300, 17), (1025,), (8, 64)], 4
    say(f"AG alignment st_off={st_off} p_off={p_off}")
    geo, S = ogeo.group_geometry(shapes, R)
    stage = normal_bf16_bits((R * S,), 1.0, 71, 0)
    want = oracle.all_gather_place(stage, shapes, R)
    for mode, launch in ((TIDE_AG_KERNEL, Launch()), (TIDE_AG_KERNEL, Launch.bounded(2)),
                         (TIDE_AG_KERNEL, Launch.cu_exclusive(3)), (TIDE_AG_SDMA, Launch()), (TIDE_AG_COPY2D, Launch())):
        got = run_ag(shapes, R, stage, mode=mode, launch=launch, st_pad=st_off,
                     p_pad=lambda p: (p_off * (p + 1)) % 8)
        for a, b in zip(got, want):
            assert np.array_equal(a, b), (mode, launch)


def test_rs_special_values(gpu_available):
    """-0.0, bf16 subnormals, +-inf, order-sensitive triples, integer sums."""
    say("special values")
    shapes, R = [(4, 8), (6,)], 2
    vals = np.array([0x8000, 0x0000, 0x0001, 0x8001, 0x3F80, 0x3380, 0x7F80, 0xFF80, 0x7F00, 0x4B80],
                    dtype=np.uint16)
    rng = np.random.default_rng(5)
    C = 5
    g = [[vals[rng.integers(0, len(vals), size=s)] for s in shapes] for _ in range(C)]
    # force the golden order case into element 0 and the all -0.0 case into element 1
    for c, b in enumerate([0x3F80, 0x3380, 0x3380, 0x0000, 0x0000]):
        g[c][0].reshape(-1)[0] = b if c < 3 else 0x0000
    for c in range(C):
        g[c][0].reshape(-1)[1] = 0x8000
    want = oracle.reduce_scatter(g, shapes, R)
    got = run_rs(shapes, R, g)
    wb = want.view(np.uint32)
    both_nan = np.isnan(want) & np.isnan(got.view(np.float32))
    assert np.array_equal(got[~both_nan], wb[~both_nan])
    assert got[0, 1] == 0x80000000


def test_rs_inputs_unchanged_and_stream(gpu_available):
    say("input immutability on a side stream")
    shapes, R, C = [(513, 9), (77,)], 3, 4
    g = [[normal_bf16_bits(s, 1.0, 72, c, p) for p, s in enumerate(shapes)] for c in range(C)]
    grads = [[dev_bf16(g[c][p]) for p in range(len(shapes))] for c in range(C)]
    before = [[host_bits_bf16(t).copy() for t in row] for row in grads]
    side = torch.cuda.Stream()
    with Layout(shapes, R) as L:
        shards = poisoned_shards(R, L.S)
        torch.cuda.synchronize()
        with torch.cuda.stream(side):
            L.rs_bf16_to_fp32(grads, shards)
        side.synchronize()
        got = np.stack([host_bits_f32(s) for s in shards])
    assert_rs_equal(got, oracle.reduce_scatter(g, shapes, R))
    for row_b, row in zip(before, grads):
        for b, t in zip(row_b, row):
            assert np.array_equal(b, host_bits_bf16(t))


def test_identical_contributor_buffers(gpu_available):
    """The same buffer passed as every contributor (inputs may alias): C * x exactly."""
    say("aliased contributors")
    shapes, R, C = [(100, 10)], 4, 8
    x = normal_bf16_bits(shapes[0], 1.0, 73, 0)
    t = dev_bf16(x)
    with Layout(shapes, R) as L:
        shards = poisoned_shards(R, L.S)
        L.rs_bf16_to_fp32([[t]] * C, shards)
        torch.cuda.synchronize()
        got = np.stack([host_bits_f32(s) for s in shards])
    assert_rs_equal(got, oracle.reduce_scatter([[x]] * C, shapes, R))


@pytest.mark.parametrize("C", [257, 1000])
@pytest.mark.parametrize("launch", [Launch.default(), Launch.bounded(3), Launch.per_cu_cap(2)], ids=str)
def test_many_contributors(gpu_available, C, launch):
    """C far beyond the compiled counts (the runtime-C kernel, blocks of 8 with a ragged last block):
    seven distinct N(0, 1) buffers passed in turn as the C contributors, so the ascending-order fp32
    sum over C terms, where every reordering changes bits, is checked against the oracle."""
    say(f"many contributors C={C} launch={launch}")
    shapes, R = [(300, 40), (1500,), (17, 3)], 8
    distinct = [[normal_bf16_bits(s, 1.0, 175, d, p) for p, s in enumerate(shapes)] for d in range(7)]
    dev = [[dev_bf16(b) for b in row] for row in distinct]
    grads = [dev[c % 7] for c in range(C)]
    with Layout(shapes, R) as L:
        shards = poisoned_shards(R, L.S)
        L.rs_bf16_to_fp32(grads, shards, launch=launch)
        torch.cuda.synchronize()
        got = np.stack([host_bits_f32(s) for s in shards])
    assert_rs_equal(got, oracle.reduce_scatter([distinct[c % 7] for c in range(C)], shapes, R))


def test_many_ranks(gpu_available):
    """R = 1000 ranks over parameters with fewer rows than ranks: ranks past the data hold padding
    only (+0.0), every shard is written in full, and the placement skips the padding."""
    say("many ranks R=1000")
    shapes, R, C = [(5000, 3), (70,), (999, 2)], 1000, 3
    bits = [[normal_bf16_bits(s, 1.0, 176, c, p) for p, s in enumerate(shapes)] for c in range(C)]
    assert_rs_equal(run_rs(shapes, R, bits), oracle.reduce_scatter(bits, shapes, R))
    with Layout(shapes, R) as L:
        S = L.S
    stage_bits = normal_bf16_bits((R * S,), 1.0, 177, 0)
    want = oracle.all_gather_place(stage_bits, shapes, R)
    for mode in (TIDE_AG_KERNEL, TIDE_AG_SDMA, TIDE_AG_COPY2D):
        got = run_ag(shapes, R, stage_bits, mode=mode)
        for g, w in zip(got, want):
            assert np.array_equal(g, w), mode


def test_overlap_rejected(gpu_available):
    shapes, R = [(64,)], 2
    g = dev_bf16(normal_bf16_bits((64,), 1.0, 74, 0))
    with Layout(shapes, R) as L:
        buf = torch.empty(64, dtype=torch.float32, device="cuda")
        with pytest.raises(TideError):
            L.rs_bf16_to_fp32([[g]], [buf[:32], buf[16:48]])


@pytest.mark.parametrize("mode", [TIDE_AG_KERNEL, TIDE_AG_SDMA, TIDE_AG_COPY2D], ids=["kernel", "sdma", "copy2d"])
def test_ag_then_rs_round_trip(gpu_available, mode):
    """AG placement then RS of that single contributor on the same stream, no host sync between:
    also checks that DMA-engine copies are ordered before the next kernel on the caller's stream."""
    say(f"AG -> RS(C=1) round trip, mode={mode}")
    shapes, R = [(7, 5), (16, 3), (1, 9), (1000, 33), (4096, 64)], 4
    geo, S = ogeo.group_geometry(shapes, R)
    stage_bits = normal_bf16_bits((R * S,), 1.0, 75, 0)
    stage = dev_bf16(stage_bits)
    params = [torch.empty(s, dtype=torch.bfloat16, device="cuda") for s in shapes]
    torch.cuda.synchronize()
    with Layout(shapes, R) as L:
        L.ag_place(stage, params, mode=mode)
        shards = poisoned_shards(R, S)
        L.rs_bf16_to_fp32([params], shards)
        torch.cuda.synchronize()
        got = np.stack([host_bits_f32(s) for s in shards])
    W = ors.widen(stage_bits).reshape(R, S).view(np.uint32)
    for gg in geo:
        for r in range(R):
            v = ogeo.valid_rows(gg.rows, gg.m, r)
            a, b, e = gg.o, gg.o + v * gg.L, gg.o + gg.e
            assert np.array_equal(got[r, a:b], W[r, a:b])
            assert np.all(got[r, b:e] == 0)


# ------------------------------------------------------------------------------------------------
# Full-size workloads (the launch configuration the benchmark times: the default launch)
# ------------------------------------------------------------------------------------------------

FULL = [c for c in ORDERED if c.name != "tiny"]


def _sample_positions(geo, S, R, n_random, rng):
    """Random (r, k) plus the first and last element of every segment (and padding)."""
    rs = list(rng.integers(0, R, n_random))
    ks = list(rng.integers(0, S, n_random))
    for g in geo:
        if g.e == 0:
            continue
        for r in range(R):
            rs += [r, r]
            ks += [g.o, g.o + g.e - 1]
    return np.array(rs, dtype=np.int64), np.array(ks, dtype=np.int64)


def _locate_many(geo, R, rs, ks):
    """Vectorised oracle geometry: (p, flat source index or -1 for padding) per sample."""
    offs = np.array([g.o for g in geo], dtype=np.int64)
    p = np.searchsorted(offs, ks, side="right") - 1
    # skip empty parameters sharing an offset: searchsorted(right)-1 picks the last with o <= k
    j = ks - offs[p]
    m = np.array([g.m for g in geo], dtype=np.int64)[p]
    L = np.array([g.L for g in geo], dtype=np.int64)[p]
    rows = np.array([g.rows for g in geo], dtype=np.int64)[p]
    v = np.clip(rows - rs * m, 0, m)
    src = np.where(j < v * L, rs * m * L + j, -1)
    return p, src


def _param_runs(geo, max_elems):
    """Runs [a, b) of consecutive parameters holding at most ~max_elems shard columns (one or more
    parameters each)."""
    runs, a, n = [], 0, 0
    for p, g in enumerate(geo):
        if p > a and n + g.e > max_elems:
            runs.append((a, p))
            a, n = p, 0
        n += g.e
    runs.append((a, len(geo)))
    return runs


def _first_mismatch(got, want):
    bad = np.nonzero(got != want)[0]
    return f"{bad.size} mismatches, first at {int(bad[0])}: got {int(got[bad[0]]):#010x} want {int(want[bad[0]]):#010x}"


def oracle_rs_every_element(shapes, R, geo, grads, shards, tag, max_elems=120_000_000):
    """Every element of every shard against the oracle's reduce-scatter.

    The oracle's per-parameter geometry depends only on the parameter's shape and R, so a run of
    consecutive parameters [a, b) is a parameter group of its own whose R shards are columns
    [o_a, o_a + sum of their e_p) of the whole group's shards.  Each run's contributor tensors are
    read back from the device (where the seeded generator drew them; the HIP path only reads them),
    reduced by the oracle on the host, and compared bit for bit, padding included.
    """
    C = len(grads)
    for a, b in _param_runs(geo, max_elems):
        lo, hi = geo[a].o, geo[b - 1].o + geo[b - 1].e
        if hi == lo:
            continue
        g_host = [[host_bits_bf16(grads[c][p]) for p in range(a, b)] for c in range(C)]
        want = oracle.reduce_scatter(g_host, shapes[a:b], R).view(np.uint32)
        del g_host
        assert want.shape == (R, hi - lo)
        for r in range(R):
            got = host_bits_f32(shards[r][lo:hi])
            if not np.array_equal(got, want[r]):
                raise AssertionError(f"{tag}: params {a}..{b - 1}, rank {r}: " + _first_mismatch(got, want[r]))
        del want


def oracle_ag_every_element(shapes, R, stage, params, tag, want=None):
    """Every element of every placed parameter against the oracle's copy-out of the stage (read back
    from the device).  Returns the oracle's parameters so that several engines can share them."""
    if want is None:
        want = oracle.all_gather_place(host_bits_bf16(stage), shapes, R)
    for p, w in enumerate(want):
        got = host_bits_bf16(params[p])
        if not np.array_equal(got, w):
            bad = int(np.count_nonzero(got != w))
            raise AssertionError(f"{tag}: parameter {p} {shapes[p]}: {bad} mismatching elements")
    return want


@pytest.mark.timeout(900)
@pytest.mark.parametrize("cfg", FULL, ids=lambda c: c.name)
def test_full_size_rs_and_ag(gpu_available, cfg):
    """The full-size workloads at the launch configuration the benchmark times (the default): every
    shard element and every placed parameter element against the oracle, bit for bit."""
    say(f"full size {cfg.name}: generating inputs")
    torch.cuda.empty_cache()
    geo, S = ogeo.group_geometry(cfg.shapes, cfg.R)
    grads = [[normal_bf16_cuda(s, cfg.sigma, cfg.cfg_id, c, p) for p, s in enumerate(cfg.shapes)]
             for c in range(cfg.C)]
    with Layout(cfg.shapes, cfg.R) as L:
        assert L.S == S
        shards = poisoned_shards(cfg.R, S)
        say(f"full size {cfg.name}: RS")
        L.rs_bf16_to_fp32(grads, shards)
        torch.cuda.synchronize()

        # (1) every element against the oracle, a run of parameters at a time
        oracle_rs_every_element(cfg.shapes, cfg.R, geo, grads, shards, cfg.name)
        say(f"full size {cfg.name}: RS every element equal to the oracle ({cfg.R} x {S})")

        # (2) a second, independent check on the device: a plain torch fp32 sum in the same order
        for p, g in enumerate(geo):
            if g.e == 0:
                continue
            acc = grads[0][p].reshape(-1).float()
            for c in range(1, cfg.C):
                acc = acc + grads[c][p].reshape(-1).float()
            for r in range(cfg.R):
                v = ogeo.valid_rows(g.rows, g.m, r)
                seg = shards[r][g.o: g.o + g.e]
                lo, hi = r * g.m * g.L, (r * g.m + v) * g.L
                assert torch.equal(seg[: v * g.L].view(torch.int32), acc[lo:hi].view(torch.int32)), (r, p)
                assert bool((seg[v * g.L:].view(torch.int32) == 0).all())
            del acc
        say(f"full size {cfg.name}: torch fixed-order sum equal")

        # the CU-exclusive launch (the setting used beside compute) gives the same shards bit for bit
        shards_x = poisoned_shards(cfg.R, S)
        L.rs_bf16_to_fp32(grads, shards_x, launch=Launch.cu_exclusive(4))
        torch.cuda.synchronize()
        for r in range(cfg.R):
            assert torch.equal(shards_x[r].view(torch.int32), shards[r].view(torch.int32)), r
        del shards_x
        say(f"full size {cfg.name}: CU-exclusive RS equal")
        del grads

        # (3) AG placement, every engine, every element against the oracle; then the round trip
        stage = normal_bf16_cuda((cfg.R * S,), cfg.sigma, cfg.cfg_id, 1 << 20, 0)
        want_p = None
        for mode, launch in ((TIDE_AG_KERNEL, Launch()), (TIDE_AG_SDMA, Launch()), (TIDE_AG_COPY2D, Launch()),
                             (TIDE_AG_KERNEL, Launch.cu_exclusive(4))):
            params = [torch.full(s, float("nan"), dtype=torch.bfloat16, device="cuda") for s in cfg.shapes]
            say(f"full size {cfg.name}: AG mode={mode} launch={launch}")
            L.ag_place(stage, params, mode=mode, launch=launch)
            torch.cuda.synchronize()
            want_p = oracle_ag_every_element(cfg.shapes, cfg.R, stage, params, f"{cfg.name} AG mode={mode}", want_p)
            if mode == TIDE_AG_KERNEL and launch == Launch():
                L.rs_bf16_to_fp32([params], shards)
                torch.cuda.synchronize()
                for r in range(cfg.R):
                    want_r = (stage[r * S:(r + 1) * S].view(torch.int16).to(torch.int32) << 16)
                    assert torch.equal(shards[r].view(torch.int32), want_r), r
                say(f"full size {cfg.name}: round trip OK")
            del params
        say(f"full size {cfg.name}: AG every element equal to the oracle (all engines)")
        del want_p
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_launch_form_does_not_change_results(gpu_available):
    say("launch-form independence")
    shapes, R, C = [(4096, 512), (2048,), (1500, 300)], 8, 8
    grads = [[normal_bf16_cuda(s, 1e-3, 80, c, p) for p, s in enumerate(shapes)] for c in range(C)]
    with Layout(shapes, R) as L:
        ref = None
        for launch in (Launch.default(), Launch.bounded(1), Launch.bounded(7), Launch.bounded(64), Launch.bounded(256),
                       Launch.bounded(1024), Launch.per_cu_cap(1), Launch.per_cu_cap(6), Launch.per_cu_cap(64),
                       *[Launch.cu_exclusive(w) for w in range(1, 9)]):
            shards = poisoned_shards(R, L.S)
            L.rs_bf16_to_fp32(grads, shards, launch=launch)
            torch.cuda.synchronize()
            got = torch.stack([s.view(torch.int32) for s in shards])
            if ref is None:
                ref = got
            else:
                assert torch.equal(got, ref), launch
        # the placement too: small budgets load two items per workgroup at a time, large ones one
        stage = normal_bf16_cuda((R * L.S,), 1.0, 81, 0)
        pref = None
        for launch in (Launch.default(), *[Launch.bounded(b) for b in (1, 7, 64, 256, 512, 513, 1024)],
                       *[Launch.cu_exclusive(w) for w in (1, 4, 8)]):
            params = [torch.full(s, POISON_BF16, dtype=torch.int16, device="cuda").view(torch.bfloat16)
                      for s in shapes]
            L.ag_place(stage, params, launch=launch)
            torch.cuda.synchronize()
            got = [q.view(torch.int16).clone() for q in params]
            if pref is None:
                pref = got
                geo, S = ogeo.group_geometry(shapes, R)
                st2 = stage.view(R, S)
                for p, g in enumerate(geo):
                    want = st2[:, g.o: g.o + g.e].reshape(R * g.m, g.L)[: g.rows].reshape(-1)
                    assert torch.equal(got[p].reshape(-1), want.view(torch.int16)), p
            else:
                assert all(torch.equal(a, b) for a, b in zip(got, pref)), launch
