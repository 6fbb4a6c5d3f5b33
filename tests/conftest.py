"""Shared pytest setup: the `gpu` marker, repo imports, seeds."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; run with -m gpu")
    config.addinivalue_line("markers", "slow: long-running CPU test")


@pytest.fixture
def rng(request):
    """Per-test numpy Generator, seeded from the test's node id (stable across runs)."""
    import zlib
    import numpy as np
    return np.random.default_rng(zlib.crc32(request.node.nodeid.encode()))
