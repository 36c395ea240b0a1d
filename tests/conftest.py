"""Test configuration: the ``gpu`` marker and shared helpers.

CPU tests (``-m "not gpu"``) pin the oracle and check the C-ABI library's
exports and host-side validation.  GPU tests compare the HIP library with the
oracle on identical seeded inputs.
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) HIP device")


@pytest.fixture(scope="session")
def orc():
    import oracle
    oracle.lib()
    return oracle
