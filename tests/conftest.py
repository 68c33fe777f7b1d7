import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    # the oracle library is compiled (if it must be) before any test opens the GPU
    import oracle
    oracle.load()
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; runs through the C ABI")
    config.addinivalue_line("markers", "slow: takes more than a few seconds on the CPU")
    config.addinivalue_line("markers", "spawns: starts another program (gcc, llvm-objdump); CPU runs only")


def pytest_collection_modifyitems(config, items):
    # A process that has opened the GPU starts no other program, and GPU tests in the same run
    # open it; where a GPU is visible (counting devices does not open it) these tests are skipped.
    import torch
    if torch.cuda.device_count() == 0:
        return
    skip = pytest.mark.skip(reason="starts another program; run where no GPU is visible")
    for item in items:
        if "spawns" in item.keywords:
            item.add_marker(skip)
