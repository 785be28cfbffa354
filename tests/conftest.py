import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs a real MI355X (runs the HIP path)")


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:  # pragma: no cover
        return False


@pytest.fixture(scope="session")
def golden_dir():
    return os.path.join(ROOT, "tests", "golden")


@pytest.fixture(autouse=True)
def no_gave_up_waits(request):
    """After every GPU test: no bounded wait of any kernel gave up in the
    workspaces the binding cached (the error word at the start of each; a
    give-up means wrong outputs).  The words are cleared for the next test."""
    yield
    if request.node.get_closest_marker("gpu") is None or not gpu_available():
        return
    import chunked_linear_scan_amd as cls
    assert cls.workspace_errors() == 0, "a kernel's bounded wait gave up"
