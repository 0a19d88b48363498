import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
if str(ROOT) not in sys.path:
    sys.path.insert(0, str(ROOT))


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs through the C ABI on the GPU)")


@pytest.fixture(scope="session")
def orc():
    from oracle.oracle import Oracle, DEFAULT_LIB, build
    if not DEFAULT_LIB.exists():
        build()
    return Oracle()
