import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_collection_modifyitems(config, items):
    # GPU tests are only meaningful where a GPU is visible; on a CPU-only host
    # they are skipped rather than failed (the driver selects them with -m gpu).
    try:
        import torch
        has_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        has_gpu = False
    if has_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


@pytest.fixture(autouse=True)
def _announce_gpu_case(request):
    # name the case on the real stderr before it touches the GPU, so a run that
    # ends abruptly still shows which case was running
    if "gpu" in request.keywords:
        sys.__stderr__.write(f"\n[gpu case] {request.node.nodeid}\n")
        sys.__stderr__.flush()
    yield
