import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


import pytest


@pytest.fixture
def announce(request):
    """Prints (unbuffered, past pytest's capture) what a GPU step is about to run."""
    import sys

    def _say(msg):
        sys.__stderr__.write(f"[{request.node.name}] {msg}\n")
        sys.__stderr__.flush()
    return _say
