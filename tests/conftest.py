import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def gpu_available():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture
def rng(request):
    """A generator of its own per test, seeded from the test's id, so that a
    test's draws do not depend on which tests ran before it."""
    import zlib

    import numpy as np
    return np.random.default_rng([12345, zlib.crc32(request.node.nodeid.encode())])
