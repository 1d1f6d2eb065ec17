import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.dirname(os.path.abspath(__file__))
for p in (ROOT, HERE):
    if p not in sys.path:
        sys.path.insert(0, p)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(autouse=True)
def _sticky_error_word_checked(request):
    """In GPU tests, every forward made through the binding waits for its
    stream and fails if the workspace's sticky error word is set (a
    single-pass wait that ran out of its poll budget)."""
    if request.node.get_closest_marker("gpu") is None:
        yield
        return
    from recurrent_vision_token_gla_amd import gla
    gla.check_errors(True)
    try:
        yield
    finally:
        gla.check_errors(False)
