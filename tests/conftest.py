import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: a full-size parity case whose fp64 oracle takes "
                                       "tens of seconds on the host")


@pytest.fixture(autouse=True)
def _announce(request):
    # Name each test before it runs so that a GPU run that dies mid-test still
    # says which case it was in.
    if request.node.get_closest_marker("gpu") is not None:
        print(f"\n[case] {request.node.nodeid}", flush=True)
    yield
