"""GPU parity of prepared calls (tide_*_prepare + tide_call_launch) and of their HIP-graph replays.

A prepared call is checked once and owns a device table of its buffers' addresses; launching it
must give bit for bit what the immediate call gives, and what the oracle gives, on whatever the
buffers hold at launch time.  The kernel paths are captured into a HIP graph on a side stream and
the graph is replayed several times, with new inputs written by eager work and host
synchronisations between the replays; every replay is checked against the oracle and against the
immediate calls.
"""
import threading

import numpy as np
import pytest
import torch

import oracle
from oracle import geometry as ogeo
from oracle import rs as ors
from all_gather_placement_amd import (Layout, TIDE_AG_COPY2D, TIDE_AG_KERNEL, TIDE_AG_SDMA, TIDE_LAUNCH_CU_EXCLUSIVE,
                                      TIDE_LAUNCH_DEFAULT, TideError,
                                      Launch, tide_rs_launch_shape)
from workloads import CONFIGS, normal_bf16_bits, normal_bf16_cuda
from tests.test_gpu_parity import (GROUPS, POISON_BF16, POISON_F32, assert_rs_equal, dev_bf16, host_bits_bf16,
                                   host_bits_f32, poisoned_shards, say, _locate_many, _sample_positions)

pytestmark = pytest.mark.gpu

MODES = [(TIDE_AG_KERNEL, "kernel"), (TIDE_AG_SDMA, "sdma"), (TIDE_AG_COPY2D, "copy2d")]


def poison_(tensors, pattern, dtype):
    for t in tensors:
        t.view(dtype).fill_(pattern)


def poisoned_params(shapes):
    return [torch.full(s, POISON_BF16, dtype=torch.int16, device="cuda").view(torch.bfloat16) for s in shapes]


def poisoned_slot(R, S):
    return torch.full((R * S,), POISON_BF16, dtype=torch.int16, device="cuda").view(torch.bfloat16)


def shards_bits(shards):
    return np.stack([host_bits_f32(s) for s in shards])


@pytest.mark.parametrize("case", range(len(GROUPS)))
def test_prepared_calls_bit_exact(gpu_available, case):
    shapes, R, C = GROUPS[case]
    say(f"prepared calls, group {case}: shapes={shapes} R={R} C={C}")
    geo, S = ogeo.group_geometry(shapes, R)
    g = [[normal_bf16_bits(s, 1.0, 110 + case, c, p) for p, s in enumerate(shapes)] for c in range(C)]
    stage_bits = normal_bf16_bits((R * S,), 1.0, 120 + case, 0)
    want_rs = oracle.reduce_scatter(g, shapes, R)
    want_ag = oracle.all_gather_place(stage_bits, shapes, R)
    want_pack = oracle.pack_slot(g[0], shapes, R)
    grads = [[dev_bf16(x) for x in row] for row in g]
    stage = dev_bf16(stage_bits)
    with Layout(shapes, R) as L:
        for launch in (Launch.default(), Launch.bounded(3), Launch.per_cu_cap(4)):
            shards = poisoned_shards(R, S)
            call = L.bind_rs(grads, shards, launch=launch)
            for _ in range(2):  # a launch rewrites every element: the second must change nothing
                call.launch()
                torch.cuda.synchronize()
                assert_rs_equal(shards_bits(shards), want_rs)
            call.close()
        for mode, name in MODES:
            params = poisoned_params(shapes)
            call = L.bind_ag(stage, params, mode=mode)
            call.launch()
            torch.cuda.synchronize()
            for a, b in zip([host_bits_bf16(q) for q in params], want_ag):
                assert np.array_equal(a, b), name
        slots = [poisoned_slot(R, S) for _ in range(C)]
        packs = [L.bind_slot_pack(grads[c], slots[c], launch=Launch.bounded(3)) for c in range(C)]
        for p in packs:
            p.launch()
        torch.cuda.synchronize()
        assert np.array_equal(host_bits_bf16(slots[0]), want_pack)
        shards = poisoned_shards(R, S)
        L.bind_rs_slots(slots, shards).launch()
        torch.cuda.synchronize()
        assert_rs_equal(shards_bits(shards), want_rs)


def test_prepared_call_reads_current_contents(gpu_available):
    """The call holds addresses, not values: new gradient values give the new sum."""
    shapes, R, C = GROUPS[1]
    say("prepared call after the inputs changed")
    geo, S = ogeo.group_geometry(shapes, R)
    with Layout(shapes, R) as L:
        grads = [[torch.empty(s, dtype=torch.bfloat16, device="cuda") for s in shapes] for _ in range(C)]
        shards = poisoned_shards(R, S)
        call = L.bind_rs(grads, shards)
        for it in range(3):
            g = [[normal_bf16_bits(s, 1.0, 130, it, c, p) for p, s in enumerate(shapes)] for c in range(C)]
            for c in range(C):
                for p in range(len(shapes)):
                    grads[c][p].copy_(dev_bf16(g[c][p]))
            call.launch()
            torch.cuda.synchronize()
            assert_rs_equal(shards_bits(shards), oracle.reduce_scatter(g, shapes, R))


def test_prepare_rejects_what_the_immediate_call_rejects(gpu_available):
    shapes, R = [(64, 8), (33,)], 4
    say("prepare argument checks")
    geo, S = ogeo.group_geometry(shapes, R)
    with Layout(shapes, R) as L:
        grads = [[torch.zeros(s, dtype=torch.bfloat16, device="cuda") for s in shapes]]
        shards = poisoned_shards(R, S)
        bad = list(shards)
        bad[1] = bad[0]  # two ranks writing one shard
        with pytest.raises(TideError, match="INVALID"):
            L.bind_rs(grads, bad)
        for bad in (Launch(9, 0), Launch(TIDE_LAUNCH_CU_EXCLUSIVE, 9), Launch(TIDE_LAUNCH_DEFAULT, 2)):
            with pytest.raises(TideError, match="INVALID"):
                L.bind_rs(grads, shards, launch=bad)  # no such form / count
        stage = torch.zeros(R * S, dtype=torch.bfloat16, device="cuda")
        params = [torch.zeros(s, dtype=torch.bfloat16, device="cuda") for s in shapes]
        with pytest.raises(TideError, match="INVALID"):
            L.bind_ag(stage, [params[0], params[0].view(-1)[: shapes[1][0]]])  # parameters overlap
        with pytest.raises(TideError, match="INVALID"):
            L.bind_ag(stage, params, mode=9)


def _capture(calls, stream):
    for c in calls:  # one eager launch first, so nothing is loaded for the first time under capture
        c.launch(stream)
    stream.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for c in calls:
            c.launch(stream)
    return g


@pytest.mark.parametrize("launch,rs_launch",
                         [(Launch(), Launch()), (Launch.bounded(3), Launch.bounded(3)),
                          (Launch.cu_exclusive(4), Launch.cu_exclusive(4)), (Launch(), Launch.per_cu_cap(6))],
                         ids=["default", "bounded3", "cu_exclusive4", "per_cu_cap6"])
def test_graph_replay_kernel_paths(gpu_available, launch, rs_launch):
    """RS, AG placement (kernel), Slot-Reuse pack + RS from slots, captured once, replayed 4 times
    (the two RS calls in rs_launch, the placement and the packing in launch)."""
    shapes, R, C = GROUPS[1]
    say(f"graph capture and replay, launch={launch} rs_launch={rs_launch}")
    geo, S = ogeo.group_geometry(shapes, R)
    with Layout(shapes, R) as L:
        grads = [[torch.empty(s, dtype=torch.bfloat16, device="cuda") for s in shapes] for _ in range(C)]
        stage = torch.empty(R * S, dtype=torch.bfloat16, device="cuda")
        shards = poisoned_shards(R, S)
        shards2 = poisoned_shards(R, S)
        params = poisoned_params(shapes)
        slots = [poisoned_slot(R, S) for _ in range(C)]
        calls = [L.bind_rs(grads, shards, launch=rs_launch), L.bind_ag(stage, params, launch=launch)]
        calls += [L.bind_slot_pack(grads[c], slots[c], launch=launch) for c in range(C)]
        calls.append(L.bind_rs_slots(slots, shards2, launch=rs_launch))
        side = torch.cuda.Stream()
        torch.cuda.synchronize()
        graph = _capture(calls, side)
        torch.cuda.synchronize()
        for it in range(4):
            g = [[normal_bf16_bits(s, 1.0, 140, it, c, p) for p, s in enumerate(shapes)] for c in range(C)]
            st = normal_bf16_bits((R * S,), 1.0, 141, it)
            for c in range(C):
                for p in range(len(shapes)):
                    grads[c][p].copy_(dev_bf16(g[c][p]))
            stage.copy_(dev_bf16(st))
            poison_(shards + shards2, POISON_F32, torch.int32)
            poison_(params + slots, POISON_BF16, torch.int16)
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            want = oracle.reduce_scatter(g, shapes, R)
            assert_rs_equal(shards_bits(shards), want)
            assert_rs_equal(shards_bits(shards2), want)
            for a, b in zip([host_bits_bf16(q) for q in params], oracle.all_gather_place(st, shapes, R)):
                assert np.array_equal(a, b), f"replay {it}"
            for c in range(C):
                assert np.array_equal(host_bits_bf16(slots[c]), oracle.pack_slot(g[c], shapes, R)), f"replay {it}"
            # eager immediate calls on the same inputs agree with the replay
            eager = poisoned_shards(R, S)
            L.rs_bf16_to_fp32(grads, eager, launch=rs_launch)
            torch.cuda.synchronize()
            assert np.array_equal(shards_bits(eager), shards_bits(shards))
        del graph
        torch.cuda.synchronize()
        for c in calls:
            c.close()


def test_graph_replay_full_size_step(gpu_available):
    """The Llama-3.1-8B layer group's step (RS from 8 contributors + AG placement) as a graph: each
    replay must equal the immediate calls bit for bit; inputs change between replays."""
    cfg = CONFIGS["llama3_1_8b_layer"]
    say(f"graph replay full size {cfg.name}")
    torch.cuda.empty_cache()
    geo, S = ogeo.group_geometry(cfg.shapes, cfg.R)
    with Layout(cfg.shapes, cfg.R) as L:
        grads = [[normal_bf16_cuda(s, cfg.sigma, cfg.cfg_id, c, p) for p, s in enumerate(cfg.shapes)]
                 for c in range(cfg.C)]
        stage = normal_bf16_cuda((cfg.R * S,), 1.0, cfg.cfg_id, 1 << 20)
        shards = [torch.empty(S, dtype=torch.float32, device="cuda") for _ in range(cfg.R)]
        params = [torch.empty(s, dtype=torch.bfloat16, device="cuda") for s in cfg.shapes]
        rs = L.bind_rs(grads, shards, launch=Launch.bounded(512))
        ag = L.bind_ag(stage, params, launch=Launch.bounded(512))
        side = torch.cuda.Stream()
        torch.cuda.synchronize()
        graph = _capture([rs, ag], side)
        torch.cuda.synchronize()
        ref_shards = [torch.empty_like(x) for x in shards]
        ref_params = [torch.empty_like(x) for x in params]
        for it in range(3):
            if it:
                for c in range(cfg.C):  # new gradients: scale every contributor's first parameter
                    grads[c][0].mul_(-0.5 if (c + it) % 2 else 2.0)
                stage.neg_()
            poison_(shards, POISON_F32, torch.int32)
            poison_(params, POISON_BF16, torch.int16)
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            L.rs_bf16_to_fp32(grads, ref_shards)
            L.ag_place(stage, ref_params)
            torch.cuda.synchronize()
            for a, b in zip(shards, ref_shards):
                assert torch.equal(a.view(torch.int32), b.view(torch.int32)), f"replay {it}"
            for a, b in zip(params, ref_params):
                assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"replay {it}"
        # sampled outputs of the last replay against the oracle, computed one by one
        rng = np.random.default_rng(cfg.cfg_id + 7)
        rs_, ks = _sample_positions(geo, S, cfg.R, 4000, rng)
        p_idx, src = _locate_many(geo, cfg.R, rs_, ks)
        got = np.empty(len(rs_), dtype=np.uint32)
        for r in range(cfg.R):
            sel = np.nonzero(rs_ == r)[0]
            if sel.size:
                got[sel] = host_bits_f32(shards[r][torch.from_numpy(ks[sel]).cuda()])
        vals = np.zeros((cfg.C, len(rs_)), dtype=np.uint16)
        for p in np.unique(p_idx):
            sel = np.nonzero((p_idx == p) & (src >= 0))[0]
            if sel.size:
                idx = torch.from_numpy(src[sel]).cuda()
                for c in range(cfg.C):
                    vals[c, sel] = host_bits_bf16(grads[c][p].reshape(-1)[idx])
        want = np.where(src >= 0, ors.rs_sampled(vals).view(np.uint32), 0).astype(np.uint32)
        assert np.array_equal(got, want), f"{int((got != want).sum())} sampled mismatches"
        del graph
        torch.cuda.synchronize()
        rs.close()
        ag.close()


def test_prepared_calls_from_threads(gpu_available):
    """One layout, four host threads, each with its own stream, buffers and prepared calls."""
    shapes, R, C = GROUPS[6]
    say("prepared calls from 4 threads")
    geo, S = ogeo.group_geometry(shapes, R)
    nthreads, iters = 4, 5
    errors = []
    with Layout(shapes, R) as L:
        work = []
        for t in range(nthreads):
            g = [[normal_bf16_bits(s, 1.0, 150, t, c, p) for p, s in enumerate(shapes)] for c in range(C)]
            st = normal_bf16_bits((R * S,), 1.0, 151, t)
            work.append(dict(g=g, st=st, grads=[[dev_bf16(x) for x in row] for row in g], stage=dev_bf16(st),
                             shards=poisoned_shards(R, S), params=poisoned_params(shapes),
                             stream=torch.cuda.Stream()))
        torch.cuda.synchronize()

        def run(w):
            try:
                with torch.cuda.stream(w["stream"]):
                    rs = L.bind_rs(w["grads"], w["shards"], launch=Launch.bounded(7))
                    ag = L.bind_ag(w["stage"], w["params"])
                    for _ in range(iters):
                        rs.launch(w["stream"])
                        ag.launch(w["stream"])
                        L.rs_bf16_to_fp32(w["grads"], w["shards"], stream=w["stream"])
                    w["stream"].synchronize()
                    rs.close()
                    ag.close()
            except Exception as e:  # reported by the main thread
                errors.append(e)

        threads = [threading.Thread(target=run, args=(w,)) for w in work]
        for th in threads:
            th.start()
        for th in threads:
            th.join()
        torch.cuda.synchronize()
        assert not errors, errors
        for w in work:
            assert_rs_equal(shards_bits(w["shards"]), oracle.reduce_scatter(w["g"], shapes, R))
            for a, b in zip([host_bits_bf16(q) for q in w["params"]], oracle.all_gather_place(w["st"], shapes, R)):
                assert np.array_equal(a, b)


def test_rs_launch_shapes(gpu_available):
    """The RS launch shape of each form (tide_rs_launch_shape) on a gfx950 CU's 160 KiB of local
    memory.  Default: CU-exclusive workgroups of 1024 threads taking 16 items (C <= 3) or 8 (C >= 4,
    the runtime-C form included) and the whole local memory; CU-exclusive N: 128*min(N, 8)
    threads, N items; per-CU cap N: single-item 128-thread workgroups requesting 1/N of it; bounded:
    128 threads, 4 items, no dynamic local memory."""
    lds_per_cu = 160 * 1024
    for C, items in ((1, 16), (2, 16), (3, 16), (4, 8), (5, 8), (7, 8), (8, 8), (9, 8), (16, 8), (17, 8), (40, 8)):
        shape = tide_rs_launch_shape(C)
        say(f"RS default launch shape C={C}: {shape}")
        assert shape == tide_rs_launch_shape(C, Launch.cu_exclusive(items)), (C, shape)
        assert shape["threads"] == 1024 and shape["items_per_workgroup"] == items and shape["item_outputs"] == 1024
        assert lds_per_cu // 2 < shape["lds_bytes"] <= lds_per_cu, (C, shape)  # one workgroup per CU
    for n in (1, 3, 8, 16):
        shape = tide_rs_launch_shape(4, Launch.cu_exclusive(n))
        assert shape["threads"] == 128 * min(n, 8) and shape["items_per_workgroup"] == n, (n, shape)
    for C in (2, 8, 20):
        b = tide_rs_launch_shape(C, Launch.bounded(5))
        assert b["threads"] == 128 and b["items_per_workgroup"] == 4 and b["lds_bytes"] < lds_per_cu // 16, b
        for n in (2, 6, 12):
            shape = tide_rs_launch_shape(C, Launch.per_cu_cap(n))
            assert shape["threads"] == 128 and shape["items_per_workgroup"] == 1
            assert shape["lds_bytes"] * n <= lds_per_cu < shape["lds_bytes"] * (n + 1), (C, n, shape)
    for C, bad in ((3, Launch(TIDE_LAUNCH_CU_EXCLUSIVE, 32)), (5, Launch.cu_exclusive(16)),
                   (1, Launch(TIDE_LAUNCH_CU_EXCLUSIVE, 24))):
        with pytest.raises(TideError, match="INVALID"):
            tide_rs_launch_shape(C, bad)


def test_rs_per_cu_cap_sets_the_cap_and_changes_speed_only(gpu_available):
    """TIDE_LAUNCH_PER_CU_CAP N: one launch with at most N RS workgroups per CU, for any C (compiled-C
    and runtime-C kernels); the shards stay bit for bit those of the oracle, immediate and prepared."""
    for shapes, R, C in (GROUPS[1], ([(300, 70), (17,), (2048, 3)], 4, 18)):
        geo, S = ogeo.group_geometry(shapes, R)
        g = [[normal_bf16_bits(s, 1.0, 160, c, p) for p, s in enumerate(shapes)] for c in range(C)]
        grads = [[dev_bf16(x) for x in row] for row in g]
        want = oracle.reduce_scatter(g, shapes, R)
        static = tide_rs_launch_shape(C, Launch.bounded(5))["lds_bytes"]  # bounded launches add none
        for n in (1, 3, 6, 16, 64):
            shape = tide_rs_launch_shape(C, Launch.per_cu_cap(n))
            say(f"RS C={C} per-CU cap {n}: {shape}")
            want_lds = max(static, (160 * 1024 // n) // 512 * 512)
            if n == 1:  # may exceed one workgroup's limit: then the smallest cap it can express
                assert static < shape["lds_bytes"] <= want_lds, shape
            else:
                assert shape["lds_bytes"] == want_lds, (n, shape)
            with Layout(shapes, R) as L:
                shards = poisoned_shards(R, S)
                L.rs_bf16_to_fp32(grads, shards, launch=Launch.per_cu_cap(n))
                torch.cuda.synchronize()
                assert_rs_equal(shards_bits(shards), want)
                shards = poisoned_shards(R, S)
                call = L.bind_rs(grads, shards, launch=Launch.per_cu_cap(n))
                call.launch()
                torch.cuda.synchronize()
                call.close()
                assert_rs_equal(shards_bits(shards), want)
        assert static < 160 * 1024 // 16


def test_rs_cu_exclusive_modes(gpu_available):
    """TIDE_LAUNCH_CU_EXCLUSIVE N: one launch of workgroups that take the largest local memory a
    workgroup may request (one per CU), N = 1..8 items (one per 128-thread group) and, where C allows,
    16 (two items' loads in flight per group).  For every N, compiled forms (C = 8, 4, 6, 2)
    and the runtime-C form (C = 18), aligned and misaligned bases, immediate and prepared calls, and
    Slot-Reuse's source addressing, the shards equal the oracle's bit for bit."""
    groups = [(GROUPS[1], 0), (([(4096, 64), (129, 7), (3,)], 8, 4), 1), (([(1000, 24), (5,), (96, 64)], 8, 6), 3),
              (([(6000, 40), (77, 9)], 4, 2), 0), (([(300, 70), (17,), (2048, 3)], 4, 18), 0)]
    for (shapes, R, C), pad in groups:
        geo, S = ogeo.group_geometry(shapes, R)
        g = [[normal_bf16_bits(s, 1.0, 190, c, p) for p, s in enumerate(shapes)] for c in range(C)]
        want = oracle.reduce_scatter(g, shapes, R)
        grads = [[dev_bf16(x, pad) for x in row] for row in g]
        with Layout(shapes, R) as L:
            slots = [poisoned_slot(R, S) for _ in range(C)]
            for c in range(C):
                L.slot_pack(grads[c], slots[c])
            ns = list(range(1, 9)) + ([16] if C <= 4 else [])
            for n in ns:
                launch = Launch.cu_exclusive(n)
                say(f"RS CU-exclusive C={C} N={n} pad={pad}: {tide_rs_launch_shape(C, launch)}")
                shards = poisoned_shards(R, S, pad)
                L.rs_bf16_to_fp32(grads, shards, launch=launch)
                torch.cuda.synchronize()
                assert_rs_equal(shards_bits(shards), want)
                if n in (1, 4, 8, 16):
                    shards = poisoned_shards(R, S, pad)
                    call = L.bind_rs(grads, shards, launch=launch)
                    call.launch()
                    torch.cuda.synchronize()
                    call.close()
                    assert_rs_equal(shards_bits(shards), want)
                    shards = poisoned_shards(R, S)
                    L.rs_slots_bf16_to_fp32(slots, shards, launch=launch)
                    torch.cuda.synchronize()
                    assert_rs_equal(shards_bits(shards), want)
    with Layout(*GROUPS[0][:2]) as L:
        shards = poisoned_shards(GROUPS[0][1], L.S)
        grads = [[torch.zeros(s, dtype=torch.bfloat16, device="cuda") for s in GROUPS[0][0]] for _ in range(4)]
        for bad in (Launch(TIDE_LAUNCH_CU_EXCLUSIVE, 9), Launch(TIDE_LAUNCH_CU_EXCLUSIVE, 32),
                    Launch(TIDE_LAUNCH_CU_EXCLUSIVE, 0)):
            with pytest.raises(TideError, match="INVALID"):
                L.rs_bf16_to_fp32(grads, shards, launch=bad)
    with pytest.raises(ValueError):
        Launch.cu_exclusive(9)


def test_ag_cu_exclusive_modes(gpu_available):
    """TIDE_LAUNCH_CU_EXCLUSIVE W for the placement kernel and Slot-Reuse packing: for every W,
    aligned and misaligned bases, immediate and prepared calls, the parameters and the packed slot equal
    the oracle's bit for bit; the DMA engines and the runtime 2-D copy reject it, and so does the
    placement any per-CU cap."""
    groups = [(GROUPS[1], 0), (GROUPS[6], 0), (([(1000, 24), (5,), (96, 64)], 8, 6), 3), (GROUPS[0], 1)]
    for (shapes, R, C), pad in groups:
        geo, S = ogeo.group_geometry(shapes, R)
        st_bits = normal_bf16_bits((R * S,), 1.0, 195, 0)
        want = oracle.all_gather_place(st_bits, shapes, R)
        g = [normal_bf16_bits(s, 1.0, 196, 0, p) for p, s in enumerate(shapes)]
        want_slot = oracle.pack_slot(g, shapes, R)
        stage = dev_bf16(st_bits, pad)
        grads = [dev_bf16(x, pad) for x in g]
        with Layout(shapes, R) as L:
            for w in range(1, 9):
                launch = Launch.cu_exclusive(w)
                say(f"AG CU-exclusive W={w} R={R} pad={pad}")
                params = poisoned_params(shapes)
                L.ag_place(stage, params, launch=launch)
                slot = poisoned_slot(R, S)
                L.slot_pack(grads, slot, launch=launch)
                torch.cuda.synchronize()
                for a, b in zip([host_bits_bf16(q) for q in params], want):
                    assert np.array_equal(a, b), (w, pad)
                assert np.array_equal(host_bits_bf16(slot), want_slot), (w, pad)
                if w in (1, 4, 8):
                    params = poisoned_params(shapes)
                    call = L.bind_ag(stage, params, launch=launch)
                    call.launch()
                    torch.cuda.synchronize()
                    call.close()
                    for a, b in zip([host_bits_bf16(q) for q in params], want):
                        assert np.array_equal(a, b), (w, pad)
            for mode in (TIDE_AG_SDMA, TIDE_AG_COPY2D):
                with pytest.raises(TideError, match="INVALID"):
                    L.ag_place(stage, poisoned_params(shapes), mode=mode, launch=Launch.cu_exclusive(4))
            for bad in (Launch.per_cu_cap(1), Launch(TIDE_LAUNCH_CU_EXCLUSIVE, 16)):
                with pytest.raises(TideError, match="INVALID"):
                    L.ag_place(stage, poisoned_params(shapes), launch=bad)


def test_destroy_with_work_in_flight(gpu_available):
    """Closing a prepared call, or a layout, right after launching (no synchronisation) is safe:
    destroy waits for the queued kernels that read the tables before freeing them."""
    shapes, R, C = GROUPS[1]
    geo, S = ogeo.group_geometry(shapes, R)
    g = [[normal_bf16_bits(s, 1.0, 180, c, p) for p, s in enumerate(shapes)] for c in range(C)]
    grads = [[dev_bf16(x) for x in row] for row in g]
    want = oracle.reduce_scatter(g, shapes, R)
    say("destroy with work in flight")
    with Layout(shapes, R) as L:
        shards = poisoned_shards(R, S)
        call = L.bind_rs(grads, shards, launch=Launch.bounded(2))  # many short launches queued
        for _ in range(3):
            call.launch()
        call.close()
        scratch = [torch.full((1 << 16,), -1, dtype=torch.int64, device="cuda") for _ in range(8)]
        torch.cuda.synchronize()
        assert_rs_equal(shards_bits(shards), want)
        del scratch
    shards = poisoned_shards(R, S)
    L = Layout(shapes, R)
    L.rs_bf16_to_fp32(grads, shards, launch=Launch.bounded(2))
    L.close()
    torch.cuda.synchronize()
    assert_rs_equal(shards_bits(shards), want)


def test_destroy_waits_for_its_own_work_only(gpu_available):
    """Destroying a prepared call, or a layout, waits for the work that reads its tables (the
    call's launches, the layout's immediate calls) and not for a kernel running on another stream:
    once the call's own work has finished, a 200 ms spin workgroup started on a side stream is still
    running when destroy returns (a device-wide wait would take the whole 200 ms).  The spin starts
    after the call's work because streams share the device's few hardware queues: work queued behind
    it in the same queue would wait for it whoever waits on that work."""
    import time

    from all_gather_placement_amd import probe as pr

    shapes, R, C = GROUPS[1]
    geo, S = ogeo.group_geometry(shapes, R)
    g = [[normal_bf16_bits(s, 1.0, 181, c, p) for p, s in enumerate(shapes)] for c in range(C)]
    grads = [[dev_bf16(x) for x in row] for row in g]
    want = oracle.reduce_scatter(g, shapes, R)
    khz = pr.wall_clock_khz()
    other = torch.cuda.Stream()
    for what in ("call", "layout"):
        say(f"destroy ({what}) beside a spin kernel on another stream")
        torch.cuda.synchronize()
        L = Layout(shapes, R)
        shards = poisoned_shards(R, S)
        call = L.bind_rs(grads, shards) if what == "call" else None
        if what == "call":
            call.launch()
        else:
            L.rs_bf16_to_fp32(grads, shards)
        torch.cuda.current_stream().synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record(other)
        pr.probe_launch(1, pr.TIDE_PROBE_SMALL, khz * 200, None, other)  # one workgroup, 200 ms
        t1.record(other)
        time.sleep(0.01)  # let the spin start
        t = time.perf_counter()
        if what == "call":
            call.close()  # waits for the call's launch (its event), not for the side stream
        else:
            L.close()  # waits for the immediate call's kernels (its table slot's event)
        waited = time.perf_counter() - t
        still_running = not t1.query()
        other.synchronize()
        spin_ms = t0.elapsed_time(t1)
        torch.cuda.synchronize()
        assert_rs_equal(shards_bits(shards), want)
        say(f"destroy ({what}): returned after {waited * 1e3:.1f} ms, the side kernel ran {spin_ms:.1f} ms")
        assert spin_ms > 100.0, spin_ms
        assert still_running and waited * 1e3 < 0.5 * spin_ms, (waited, spin_ms)
        L.close()


def test_closing_the_layout_closes_its_calls(gpu_available):
    """Prepared calls address their layout's tables: closing the layout closes them, and a later
    launch raises instead of reading freed memory."""
    shapes, R, C = GROUPS[0]
    geo, S = ogeo.group_geometry(shapes, R)
    grads = [[torch.zeros(s, dtype=torch.bfloat16, device="cuda") for s in shapes] for _ in range(C)]
    shards = poisoned_shards(R, S)
    say("layout close closes its calls")
    L = Layout(shapes, R)
    call = L.bind_rs(grads, shards)
    call.launch()
    L.close()
    with pytest.raises(TideError, match="closed"):
        call.launch()
    torch.cuda.synchronize()
    assert np.all(shards_bits(shards) == 0)  # the launch before the close completed: all +0.0
