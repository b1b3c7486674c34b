import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


import pytest  # noqa: E402


@pytest.fixture
def kve_overrides():
    """Set the library's test overrides for one test; reset to the defaults after it."""
    import decode_kv_cache_evict_amd as kv
    state = {"score_impl": "default", "spin_limit": 0}

    def set_(**kw):
        state.update(kw)
        kv.kve_set_test_overrides(state["score_impl"], state["spin_limit"])

    yield set_
    kv.kve_set_test_overrides("default", 0)
