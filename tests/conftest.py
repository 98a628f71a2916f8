"""Shared test configuration.

Markers:
  gpu  — needs an MI355X (gfx950) and the built HIP library; run with -m gpu.
Everything else runs on the CPU.
"""
import os
import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parent.parent
if str(ROOT) not in sys.path:
    sys.path.insert(0, str(ROOT))


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU test")


@pytest.fixture(scope="session")
def oracle_mod():
    import oracle
    oracle.default()
    return oracle
