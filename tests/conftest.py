import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_collection_modifyitems(config, items):
    # GPU tests fail loudly (not skip) when the marker is selected but no GPU is
    # present: a silent skip would hide a missing device on the GPU machine.
    pass


@pytest.fixture(scope="session")
def golden_blocks():
    from tests.golden_blocks import load_golden_blocks
    return load_golden_blocks()
