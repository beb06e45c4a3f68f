import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_runtest_setup(item):
    # Name the case on the real stderr before it runs, so a run that dies on
    # the GPU still shows which test was in flight.
    if item.get_closest_marker("gpu") is not None:
        sys.__stderr__.write(f"[gpu-case] {item.nodeid}\n")
        sys.__stderr__.flush()
