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
