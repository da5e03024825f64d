import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "timeout(seconds): per-test time limit (pytest-timeout)")


_HAS_GPU = None


def _has_gpu():
    global _HAS_GPU
    if _HAS_GPU is None:
        import torch
        _HAS_GPU = torch.cuda.is_available()
    return _HAS_GPU


def pytest_runtest_setup(item):
    if item.get_closest_marker("gpu") is not None and not _has_gpu():
        pytest.skip("no GPU on this machine")
