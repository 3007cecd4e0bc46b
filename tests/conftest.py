"""Shared test configuration.

``gpu`` marks tests that need an MI355X (gfx950) GPU; they are skipped where no GPU is
visible.  Everything else runs on the CPU.
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; skipped without one")
    config.addinivalue_line("markers", "slow: long-running CPU test")


_gpu = None


def gpu_available() -> bool:
    global _gpu
    if _gpu is None:
        try:
            import torch
            _gpu = bool(torch.cuda.is_available())
        except Exception:
            _gpu = False
    return _gpu


def pytest_collection_modifyitems(config, items):
    for item in items:
        if "gpu" in item.keywords and not gpu_available():
            item.add_marker(pytest.mark.skip(reason="no GPU visible"))
