import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs through the HIP library)")
    config.addinivalue_line("markers", "slow: long CPU test")


@pytest.fixture(autouse=True)
def device_checks(request):
    """With the debug build loaded (KVSEL_LIBRARY naming libkvsel_debug.so),
    every GPU test ends by reading the kernels' device-side check counts: a
    failed check fails the test that ran it."""
    yield
    if request.node.get_closest_marker("gpu") is None:
        return
    if not os.environ.get("KVSEL_LIBRARY", "").endswith("libkvsel_debug.so"):
        return
    import torch
    from decode_focal_layer_amd import kvsel
    torch.cuda.synchronize()
    st, n, code, detail = kvsel.debug_status()
    assert st == 0, f"{n} device check(s) failed; first: code {code}, detail {detail}"
