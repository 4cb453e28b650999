import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


import pytest  # noqa: E402


@pytest.fixture(autouse=True)
def _device_status_words(request):
    """After every GPU test: no SGMM workspace a test used may report a wait that gave up
    (its outputs would be invalid) or an out-of-range adapter index (rp_workspace_status)."""
    yield
    if request.node.get_closest_marker("gpu") is None:
        return
    import rank_pregate_amd as rp
    if rp._lib is None:
        return
    rp.check_workspaces(clear=True)
