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


@pytest.fixture(autouse=True)
def _debug_bounds_flags(request):
    """With the bounds-checked library (KVE_LIB=.../libkvevict_debug.so), every
    GPU test must end with no kernel index outside its segment: the flags are
    cleared before the test and must read zero after it."""
    if request.node.get_closest_marker("gpu") is None:
        yield
        return
    import decode_kv_cache_evict_amd as kv
    if os.path.basename(kv.LIB_PATH) != "libkvevict_debug.so":
        yield
        return
    kv.kve_debug_flags()
    yield
    flags = kv.kve_debug_flags()
    assert flags == 0, f"bounds checks fired: flags 0x{flags:x}"
