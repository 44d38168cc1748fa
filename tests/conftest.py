"""Shared pytest configuration: the ``gpu`` marker and import paths.

Tests marked ``gpu`` need an MI355X (gfx950).  Without a visible GPU they
are skipped; with one, a missing HIP library, or one built from other
sources than the tree's (its compiled-in fp8_source_hash differs from the
hash of scaled_quantize_fp8_amd/csrc and include/fp8linear.h), makes every
one of them fail: the product has no CPU fallback, and a stale library would
test other code than the tree holds.
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


_LIB_STATE = {}


def _library_problem():
    """None if the built library matches the tree's sources, else why not."""
    if "problem" not in _LIB_STATE:
        try:
            import scaled_quantize_fp8_amd as F
            from scaled_quantize_fp8_amd import _build
            built, tree = F.fp8_source_hash(), _build.source_hash()
            _LIB_STATE["problem"] = (None if built == tree else
                                     f"libfp8linear.so was built from other sources "
                                     f"(library {built[:12]}, tree {tree[:12]}): rebuild it")
        except Exception as exc:  # missing library or symbol
            _LIB_STATE["problem"] = f"HIP library unusable: {exc}"
    return _LIB_STATE["problem"]


@pytest.fixture(autouse=True)
def _fresh_library(request):
    if "gpu" in request.keywords and _gpu_visible():
        problem = _library_problem()
        if problem:
            pytest.fail(problem)
    yield


def pytest_collection_modifyitems(config, items):
    if _gpu_visible():
        return
    skip = pytest.mark.skip(reason="no GPU visible (needs MI355X / gfx950)")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)
