import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


@pytest.fixture(scope="session")
def golden_dir():
    return os.path.join(ROOT, "tests", "golden")


_WORKLOADS = {}


@pytest.fixture(scope="session")
def workload_cache():
    """Seeded host inputs of the named full-size workload, generated once."""
    from fmha_fwd_amd import workloads as W

    def get(name):
        if name not in _WORKLOADS:
            _WORKLOADS.clear()  # keep one full-size workload in memory at a time
            _WORKLOADS[name] = W.generate(W.SPECS[name])
        return _WORKLOADS[name]
    return get
