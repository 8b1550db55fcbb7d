"""Shared pytest set-up: repo root on sys.path and the ``gpu`` marker.

Tests marked ``gpu`` need an MI355X (gfx950) and the built HIP library; they
are skipped with a reason on a host without a visible GPU.  Everything else
runs on the CPU.
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs a visible MI355X GPU and the built HIP library")


def _gpu_visible() -> bool:
    try:
        import torch
        return bool(torch.cuda.is_available())
    except Exception:  # pragma: no cover - torch import problems
        return False


def pytest_collection_modifyitems(config, items):
    if _gpu_visible():
        return
    skip = pytest.mark.skip(reason="no visible GPU on this host")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)
