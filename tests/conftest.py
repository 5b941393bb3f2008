import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD GPU (MI355X / gfx950) and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def pytest_collection_modifyitems(config, items):
    # Run GPU tests only where a device is actually present; on a CPU-only host
    # they are skipped with a reason instead of failing at import.
    have_gpu = None
    for item in items:
        if "gpu" in item.keywords:
            if have_gpu is None:
                try:
                    import torch
                    have_gpu = torch.cuda.is_available()
                except Exception:
                    have_gpu = False
            if not have_gpu:
                item.add_marker(pytest.mark.skip(reason="no GPU visible"))
