"""Shared test set-up: repo root on sys.path and the ``gpu`` marker."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs through the HIP C-ABI library)")
    config.addinivalue_line("markers", "slow: long CPU-only check (still part of the default run)")


@pytest.fixture(scope="session")
def orc():
    """The CPU oracle's ctypes handle (built on first use)."""
    import oracle

    return oracle.load()
