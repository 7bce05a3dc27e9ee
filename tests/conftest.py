import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running test")


def gpu_visible() -> bool:
    """Whether torch sees a GPU (counting devices does not initialize one)."""
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return False


# environment that hides every GPU from HIP and the ROCm runtime
HIDE_GPUS = {"HIP_VISIBLE_DEVICES": "-1", "CUDA_VISIBLE_DEVICES": "-1",
             "ROCR_VISIBLE_DEVICES": "-1"}


def golden_path(name: str) -> str:
    return os.path.join(GOLDEN, name)


def golden_lines(name: str):
    """Non-comment, non-empty lines of a golden fixture, split on whitespace."""
    with open(golden_path(name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                yield line.split()


@pytest.fixture(scope="session")
def golden():
    return golden_lines
