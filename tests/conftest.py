import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
TESTS = os.path.dirname(os.path.abspath(__file__))
if TESTS not in sys.path:
    sys.path.insert(0, TESTS)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_collection_modifyitems(config, items):
    have_gpu = None
    for item in items:
        if "gpu" not in item.keywords:
            continue
        if have_gpu is None:
            import torch
            have_gpu = torch.cuda.is_available()
        if not have_gpu:
            item.add_marker(pytest.mark.skip(reason="no GPU visible"))
