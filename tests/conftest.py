"""Shared pytest configuration.

Markers:
  gpu  -- needs an MI355X (gfx950) and the built HIP library; parity of the
          HIP path against the float64 oracle.  Everything else runs on CPU.
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X GPU and the built HIP library")


@pytest.fixture(scope="session")
def rng():
    import numpy as np
    return np.random.default_rng(12345)
