import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


@pytest.fixture(scope="session", autouse=True)
def _native_helpers_built():
    """The generator and the oracle are plain host C; build them if absent."""
    from gated_linear_recurrence_history_amd import _build
    import oracle.build as ob
    if not os.path.exists(os.path.join(_build.PKG, "libgscan_synth.so")):
        _build.build_synth()
    if not os.path.exists(os.path.join(ROOT, "oracle", "liboracle.so")):
        ob.build()
    yield
