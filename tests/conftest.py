"""Shared pytest configuration.

Tests marked ``gpu`` need a ROCm device and the built HIP library; everything
else runs on the CPU (oracle pins, host-side validation, symbol checks).
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) device and the built libpa.so")
    config.addinivalue_line("markers", "slow: long-running; still part of the default run")


@pytest.fixture(scope="session")
def oracle_lib():
    import oracle

    oracle._load()
    return oracle


@pytest.fixture(autouse=True)
def _guard_bands(request):
    """After every GPU test: the canaries around every device buffer it handed to the
    library (tests/_gpu_helpers.py, guarded_*) must be intact."""
    yield
    if request.node.get_closest_marker("gpu") is None:
        return
    from _gpu_helpers import check_guards

    check_guards()
