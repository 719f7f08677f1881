import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; run with -m gpu")


def _gpu_visible() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def pytest_collection_modifyitems(config, items):
    markexpr = config.getoption("-m") or ""
    asked_for_gpu = "gpu" in markexpr and "not gpu" not in markexpr
    if asked_for_gpu or _gpu_visible():
        return  # GPU tests run (and fail loudly if the device is missing)
    skip = pytest.mark.skip(reason="no GPU visible; GPU tests run with -m gpu on an MI355X")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)
