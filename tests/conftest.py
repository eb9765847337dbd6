import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(autouse=True)
def _announce(request):
    # a GPU case names itself on the real stderr (past pytest's capture)
    # before it runs, so a run that ends abruptly still shows which case it was
    if request.node.get_closest_marker("gpu") is not None:
        sys.__stderr__.write("[gpu-case] %s\n" % request.node.nodeid)
        sys.__stderr__.flush()
    yield
