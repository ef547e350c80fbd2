import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# Every device workspace the binding allocates starts as 0xFF bytes (e4m3 NaN, int32 -1), so a
# kernel that reads a workspace byte no kernel of the call wrote changes its results.
os.environ.setdefault("QMOE_POISON_WORKSPACE", "1")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session", autouse=True)
def _host_libs():
    """Build the two plain-C host libraries (input generator and oracle) if missing."""
    from synth import synth
    from oracle import oracle
    synth.build()
    oracle.build()
    yield
