import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs a real MI355X (gfx950) and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workloads (seconds to minutes)")
    # Load what is built; build only when nothing is (hipcc cross-compiles without a GPU).
    from all_gather_placement_amd.build import ensure_built

    ensure_built()


def golden_path(name: str) -> str:
    return os.path.join(ROOT, "tests", "golden", name)


@pytest.fixture(scope="session")
def gpu_available():
    import torch

    # GPU tests run only where a GPU is expected: a missing device is an error, not a skip.
    assert torch.cuda.is_available(), "GPU test selected but torch sees no GPU"
    return True
