import os
import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
if str(ROOT) not in sys.path:
    sys.path.insert(0, str(ROOT))


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs the HIP library)")
    config.addinivalue_line("markers", "slow: long-running (large shapes)")


@pytest.fixture(scope="session")
def gpu():
    """A visible GPU and the loaded HIP library; fails loudly without them."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test selected but no GPU is visible")
    import invariant_rmsnorm_amd as irn
    irn.load()  # raises if the HIP library is missing
    return torch.device("cuda:0")
