import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_collection_modifyitems(config, items):
    # a GPU test without a GPU is skipped rather than failed when run unfiltered
    try:
        import torch
        has_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        has_gpu = False
    if has_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU in this environment")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


def pytest_sessionstart(session):
    # the HIP library is loaded from the tree; build it only when it is missing
    lib = os.path.join(ROOT, "paged_kv_extend_amd", "libpkv.so")
    if not os.path.exists(lib):
        from paged_kv_extend_amd import _build
        _build.build()
