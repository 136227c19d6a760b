import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU; runs the HIP library through its C ABI")
    config.addinivalue_line(
        "markers", "slow: long CPU check, run only when ZERO_EXHAUSTIVE=1")


def pytest_collection_modifyitems(config, items):
    if os.environ.get("ZERO_EXHAUSTIVE") == "1":
        return
    skip = pytest.mark.skip(reason="exhaustive check; set ZERO_EXHAUSTIVE=1 to run")
    for item in items:
        if "slow" in item.keywords:
            item.add_marker(skip)


@pytest.fixture(scope="session")
def orc():
    import oracle
    oracle.lib()
    return oracle
