import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: large shapes")


@pytest.fixture(scope="session", autouse=True)
def _build_host_libs():
    # host-side helpers (seeded generator, float64 oracle) compile in seconds
    import hils_synth
    import oracle
    hils_synth.build()
    oracle.build()
    yield
