import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built libprism.so")
    config.addinivalue_line("markers", "slow: large-shape test")


@pytest.fixture(autouse=True)
def _no_wait_giveups(request):
    """After every GPU test: no bounded in-kernel wait of the scan gave up
    (a give-up is counted on the device; the count is read and reset here)."""
    yield
    if request.node.get_closest_marker("gpu") is None:
        return
    try:
        import torch
    except ImportError:
        return
    if not torch.cuda.is_available():
        return
    from gated_delta_rule_prologue_amd import binding
    torch.cuda.synchronize()
    assert binding.scan_wait_giveups(reset=True) == 0, "a bounded scan wait gave up"
