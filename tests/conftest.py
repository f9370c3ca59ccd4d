import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: generates the large synthetic configs")


_CACHE = {}


def load_config(k):
    """Synthetic config k, generated once per test session."""
    import pzinputs

    if k not in _CACHE:
        _CACHE[k] = pzinputs.config(k)
    return _CACHE[k]


@pytest.fixture(scope="session")
def config_tensors():
    return load_config
