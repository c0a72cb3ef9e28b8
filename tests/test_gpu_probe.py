"""The occupancy probe records sane locations and times (GPU)."""
import numpy as np
import pytest
import torch

from all_gather_placement_amd import probe as pr

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("shape", [pr.TIDE_PROBE_GEMM_SHAPED, pr.TIDE_PROBE_SMALL], ids=["gemm_shaped", "small"])
def test_probe_records(gpu_available, shape):
    khz = pr.wall_clock_khz()
    assert khz > 0
    tpu = khz / 1000.0
    n = 256
    recs = torch.zeros(n * 4, dtype=torch.int64, device="cuda")
    pr.probe_launch(n, shape, int(50 * tpu), recs)
    torch.cuda.synchronize()
    d = pr.decode(recs.cpu().numpy().view(np.uint64))
    assert np.all(d["end"] >= d["start"])
    dur_us = (d["end"] - d["start"]) / tpu
    assert np.all(dur_us >= 49.0) and np.all(dur_us < 50_000)
    assert np.all(d["xcc"] < 8)
    if shape == pr.TIDE_PROBE_GEMM_SHAPED:
        # 64 KiB of LDS and 256 VGPRs per wave: alone on the device, one workgroup per CU in one wave
        assert len(np.unique(d["cu_key"])) == n
        assert (d["start"].max() - d["start"].min()) / tpu < 20.0


def test_clock_probe_reads_a_shader_clock(gpu_available):
    """The clock probe's cycle count over 1 ms of wall clock is a shader clock in the range an MI355X
    runs at (idle or busy), and its wall-clock interval covers the requested sleep."""
    khz = pr.wall_clock_khz()
    out = torch.zeros(4, dtype=torch.int64, device="cuda")
    pr.clock_probe(khz, out)  # 1 ms
    torch.cuda.synchronize()
    w0, w1, c0, c1 = out.cpu().tolist()
    assert w1 - w0 >= khz and c1 > c0
    mhz = pr.clock_mhz([w0, w1, c0, c1], khz)
    print(f"[gpu-probe] shader clock over 1 ms: {mhz:.0f} MHz", flush=True)
    assert 100.0 < mhz < 3000.0


def test_mix_probe_modes(gpu_available):
    """The mix probe in the RS's access shape: both = the oracle's ordered fp32 sums bit for bit
    (24 items, not a multiple of the 8 XCD ranges, so every item is mapped exactly once); writes only
    = its pattern in every item; reads only = no store at all."""
    import oracle
    from workloads import normal_bf16_bits

    items, C = 24, 4
    n = items * 1024
    bits = [[normal_bf16_bits((n,), 1.0, 170, c, 0)] for c in range(C)]
    grads = [torch.from_numpy(b[0].view(np.int16).copy()).cuda().view(torch.bfloat16) for b in bits]
    src = torch.tensor([g.data_ptr() for g in grads], dtype=torch.int64, device="cuda")
    want = oracle.reduce_scatter(bits, [(n,)], 1)[0].view(np.uint32)
    dst = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
    pr.mix_launch(C, pr.TIDE_PROBE_MIX_BOTH, src, dst, items, 0)
    torch.cuda.synchronize()
    assert np.array_equal(dst.view(torch.int32).cpu().numpy().view(np.uint32), want)

    dst.fill_(float("nan"))
    pr.mix_launch(C, pr.TIDE_PROBE_MIX_READS, src, dst, items, 27136)
    torch.cuda.synchronize()
    assert torch.isnan(dst).all()

    pr.mix_launch(C, pr.TIDE_PROBE_MIX_WRITES, None, dst, items, 27136)
    torch.cuda.synchronize()
    got = dst.cpu().numpy().reshape(items, 2, 128, 4)  # item, store, lane, 4 floats
    lanes = np.arange(128, dtype=np.float32)
    for st, tail in ((0, (1.0, 2.0, 3.0)), (1, (4.0, 5.0, 6.0))):
        assert np.array_equal(got[:, st, :, 0], np.broadcast_to(lanes, (items, 128)))
        for j, v in enumerate(tail):
            assert np.all(got[:, st, :, j + 1] == v)


def test_cu_mask_stream_confines_work_and_keeps_results(gpu_available):
    """A stream masked to K CUs runs its workgroups on at most K distinct CUs (disjoint from the
    complementary mask's), and an RS launched on it equals the same RS on torch's stream bit for bit."""
    from all_gather_placement_amd import Layout
    from workloads import normal_bf16_cuda

    n_cus = torch.cuda.get_device_properties(0).multi_processor_count
    khz = pr.wall_clock_khz()
    shapes, R, C = [(3000, 64), (257,)], 8, 8
    grads = [[normal_bf16_cuda(s, 1e-3, 171, c, p) for p, s in enumerate(shapes)] for c in range(C)]
    for k in (8, 64):
        s_in, h_in = pr.cu_mask_stream(0, k)
        s_out, h_out = pr.cu_mask_stream(k, n_cus - k)
        try:
            keys = []
            for st, n_wgs in ((s_in, 8 * k), (s_out, 8 * (n_cus - k))):
                recs = torch.zeros(n_wgs * 4, dtype=torch.int64, device="cuda")
                pr.probe_launch(n_wgs, pr.TIDE_PROBE_SMALL, khz // 50, recs, st)  # 20 us each
                torch.cuda.synchronize()
                keys.append(set(pr.decode(recs.cpu().numpy().view(np.uint64))["cu_key"].tolist()))
            print(f"[gpu-probe] mask of {k} CUs: workgroups on {len(keys[0])} CUs; complement on {len(keys[1])}",
                  flush=True)
            assert 0 < len(keys[0]) <= k
            assert 0 < len(keys[1]) <= n_cus - k
            assert not (keys[0] & keys[1])
            with Layout(shapes, R) as L:
                ref = [torch.full((L.S,), float("nan"), device="cuda") for _ in range(R)]
                got = [torch.full((L.S,), float("nan"), device="cuda") for _ in range(R)]
                L.rs_bf16_to_fp32(grads, ref)
                torch.cuda.synchronize()
                call = L.bind_rs(grads, got)
                call.launch(s_in)
                torch.cuda.synchronize()
                call.close()
                for a, b in zip(ref, got):
                    assert torch.equal(a.view(torch.int32), b.view(torch.int32))
        finally:
            torch.cuda.synchronize()
            pr.destroy_stream(h_in)
            pr.destroy_stream(h_out)


def test_dma_rect_copies_place_a_group_like_the_oracle(gpu_available):
    """The DMA engines' rectangular copy, one per parameter plus one per partly padded rank (the
    placement shape of bench.py --dma-rect), lands every parameter element as the oracle's copy-out."""
    import oracle
    from all_gather_placement_amd import Layout
    from bench import rect_plan
    from workloads import normal_bf16_bits

    shapes, R = [(64, 8), (33, 6), (16,), (3, 2, 4)], 4  # every slice and offset a whole 4-byte word
    with Layout(shapes, R) as L:
        stage_bits = normal_bf16_bits((R * L.S,), 1.0, 250, 0)
        stage = torch.from_numpy(stage_bits.view(np.int16).copy()).cuda().view(torch.bfloat16)
        params = [torch.full(s, -1, dtype=torch.int16, device="cuda").view(torch.bfloat16) for s in shapes]
        rects = rect_plan(L, stage, params)
        assert len(rects) == 5  # (33, 6) has a partly padded rank: 33 rows = 3 full slices of 9 + 6
        torch.cuda.synchronize()
        us = pr.dma_rect_copies(rects)
        assert us > 0
        want = oracle.all_gather_place(stage_bits, shapes, R)
        for q, w in zip(params, want):
            assert np.array_equal(q.view(torch.int16).cpu().numpy().view(np.uint16), w)
