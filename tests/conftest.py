import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parent.parent
for p in (str(ROOT), str(Path(__file__).resolve().parent)):
    if p not in sys.path:
        sys.path.insert(0, p)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long CPU test")


@pytest.fixture(scope="session")
def orc():
    import oracle
    return oracle.default()


@pytest.fixture(autouse=True)
def _announce_gpu_test(request):
    """Name each GPU test on stdout before it touches the device."""
    if request.node.get_closest_marker("gpu") is not None:
        print(f"\n[gpu] {request.node.nodeid}", file=sys.__stdout__, flush=True)
    yield
