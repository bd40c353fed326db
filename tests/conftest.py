import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; runs the HIP path through the C ABI")
    config.addinivalue_line("markers", "slow: full-size workload (seconds to minutes)")


@pytest.fixture(scope="session", autouse=True)
def _native_libs():
    """Load what is built; build the CPU-side libraries only if nothing is."""
    import oracle
    import workloads
    oracle.lib()
    workloads.lib()
