import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


import pytest


@pytest.fixture(scope="session", autouse=True)
def poisoned_workspaces():
    """Every workspace the binding allocates is filled with 0xFF bytes (NaN as
    fp16 and fp32) before each call, so a kernel that reads workspace memory it
    did not write first shows up as a non-finite or wrong result."""
    import gated_delta_rule_02_amd as gdn
    gdn.poison_workspace(True)
    yield
    gdn.poison_workspace(False)
