import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size parity case")


def pytest_collection_modifyitems(config, items):
    """GPU tests skip themselves (with the reason) when no GPU is visible."""
    try:
        import torch
        have_gpu = torch.cuda.is_available()
    except Exception:
        have_gpu = False
    if have_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for it in items:
        if "gpu" in it.keywords:
            it.add_marker(skip)


@pytest.fixture
def progress(request):
    """Print a progress line at once, past pytest's output capture: full-size
    cases run for minutes, and their steps should be visible while they do."""
    capman = request.config.pluginmanager.getplugin("capturemanager")

    def emit(msg):
        if capman is None:
            print(msg, flush=True)
            return
        with capman.global_and_fixture_disabled():
            print(msg, flush=True)
    return emit
