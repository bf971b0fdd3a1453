import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_runtest_setup(item):
    # name the case before any GPU work starts, so a run that dies on the GPU says where
    if item.get_closest_marker("gpu") is not None:
        print(f"\n[gpu-test] {item.nodeid}", flush=True)
