import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running (7B-shaped) GPU case")


def pytest_collection_modifyitems(config, items):
    """Print the test id before each GPU test starts, so a run that dies on the GPU names its case."""
    return None


def pytest_runtest_logstart(nodeid, location):
    if "gpu" in nodeid or "test_gpu" in nodeid:
        print(f"\n[start] {nodeid}", flush=True)
