import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: generates the large synthetic workloads")


_CACHE = {}


def load_workload(name):
    """The named synthetic workload, generated once per test session."""
    import pzinputs

    if name not in _CACHE:
        _CACHE[name] = pzinputs.workload(name)
    return _CACHE[name]


@pytest.fixture(scope="session")
def workload_tensors():
    return load_workload
