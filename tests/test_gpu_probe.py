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
