import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs through the HIP C-ABI)")


@pytest.fixture(scope="session")
def oracle_mod():
    import oracle
    return oracle


@pytest.fixture(autouse=True)
def _read_scan_error_words(request):
    """GPU tests: every backward and linear-scan call made through layer.py
    reads its workspace's error word afterwards and fails if it is set."""
    if request.node.get_closest_marker("gpu") is None:
        yield
        return
    from parallelizable_recurrent_units_amd import layer
    layer.CHECK_SCAN_ERRORS = True
    try:
        yield
    finally:
        layer.CHECK_SCAN_ERRORS = False
