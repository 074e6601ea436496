import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU test (full-size oracle work)")


def pytest_collection_modifyitems(config, items):
    # GPU tests print the case they run before touching the device, so a fault names it.
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(pytest.mark.timeout(300))
