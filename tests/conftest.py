"""Shared pytest configuration: the ``gpu`` marker and import paths.

Tests marked ``gpu`` need an MI355X (gfx950).  Without a visible GPU they
are skipped; with one, a missing or stale HIP library makes them fail (the
product has no CPU fallback).
"""

import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def _gpu_visible() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def pytest_collection_modifyitems(config, items):
    if _gpu_visible():
        return
    skip = pytest.mark.skip(reason="no GPU visible (needs MI355X / gfx950)")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)
