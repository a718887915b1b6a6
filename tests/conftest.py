"""Test configuration: the ``gpu`` marker and shared fixtures.

Tests marked ``gpu`` need an MI355X (gfx950) and call the HIP library through
its C ABI.  On a machine without a GPU they are skipped; everything else runs
on the CPU.
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X GPU and the built HIP library")


def pytest_sessionstart(session):
    """Tie the library under test to the source tree: a libfp8w8a8.so that is
    missing, or was built from other sources (the hash it records differs),
    is rebuilt before any test loads it."""
    from fp8_w8a8_quantized_amd import build

    if not build.is_current():
        print("libfp8w8a8.so missing or built from other sources: rebuilding", flush=True)
        build.build()


def _gpu_present() -> bool:
    try:
        import torch

        return torch.cuda.is_available() and torch.cuda.device_count() > 0
    except Exception:
        return False


def pytest_collection_modifyitems(config, items):
    if _gpu_present():
        return
    skip = pytest.mark.skip(reason="no GPU in this environment")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)
