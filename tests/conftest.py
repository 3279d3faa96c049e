"""Shared pytest configuration.

Markers: ``gpu`` marks tests that need an MI355X (they call the HIP library
through its C ABI); everything else runs on the CPU.
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
TESTS = os.path.dirname(os.path.abspath(__file__))
if TESTS not in sys.path:
    sys.path.insert(0, TESTS)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD MI355X (gfx950) GPU")


@pytest.fixture(scope="session")
def oracle_mod():
    import oracle

    if not os.path.exists(oracle.lib_path()):
        oracle.build(force=False)
    return oracle
