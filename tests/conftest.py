import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) and the built HIP library")


@pytest.fixture(scope="session")
def gpu_lib():
    """The built library, loaded through its Python binding, on cuda:0."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test collected on a machine without a GPU")
    import muon_newton_schulz_03_amd as m
    m.load_library()
    return m


@pytest.fixture(autouse=True)
def output_guards(request):
    """GPU tests: after the test, every buffer made by gpu_util.padded() must
    still hold its fill in the guard rows around the view and in the pitch
    padding (nothing was written outside an output)."""
    if request.node.get_closest_marker("gpu") is None:
        yield
        return
    import gpu_util
    gpu_util.clear_guards()
    yield
    import torch
    torch.cuda.synchronize()
    gpu_util.check_guards()
