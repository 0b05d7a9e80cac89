"""Shared pytest setup: repository root on sys.path and the ``gpu`` marker."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_collection_modifyitems(config, items):
    """GPU tests need a visible GPU; without one (a CPU-only host) they are
    skipped. With a GPU present, a missing HIP library fails them loudly."""
    if not any("gpu" in item.keywords for item in items):
        return
    import pytest
    import torch
    if torch.cuda.is_available():
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)
