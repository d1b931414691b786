import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running (full-size workload)")


@pytest.fixture(scope="session", autouse=True)
def _host_libs():
    """Build the generator and the oracle if they are not built yet (gcc, seconds)."""
    import oracle
    import synth
    if not os.path.exists(synth._SO):
        synth.build()
    if not os.path.exists(oracle._SO):
        oracle.build()
    import sparse_mixture_experts_30_amd._lib as L
    if not os.path.exists(L.SO_PATH):
        from sparse_mixture_experts_30_amd import build
        build.build()
    yield
