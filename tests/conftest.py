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
