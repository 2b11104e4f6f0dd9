import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_collection_modifyitems(config, items):
    # GPU tests fail loudly (not skip) when the device or library is missing,
    # so a `-m gpu` run on a machine without them cannot pass silently.
    pass


@pytest.fixture(scope="session")
def rng():
    import numpy as np
    return np.random.default_rng(12345)
