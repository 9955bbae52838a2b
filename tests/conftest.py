"""Shared pytest setup: repo root on sys.path, the ``gpu`` marker, GPU skips."""

import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def _has_gpu():
    try:
        import torch

        return torch.cuda.is_available()
    except Exception:  # pragma: no cover
        return False


def pytest_collection_modifyitems(config, items):
    if _has_gpu():
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


def pytest_sessionfinish(session, exitstatus):
    """Write the GPU tests' per-case accuracy records when PA_ACCURACY_REPORT names a file."""
    path = os.environ.get("PA_ACCURACY_REPORT")
    if not path:
        return
    mod = sys.modules.get("tests.gpu_util")
    recs = getattr(mod, "ACCURACY", []) if mod else []
    if not recs:
        return
    import json

    with open(path, "w") as f:
        json.dump(recs, f, indent=1)
