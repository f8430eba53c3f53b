import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_report_header(config):
    return f"repo root: {ROOT}"


@pytest.fixture(autouse=True)
def _flush_case_name(request):
    # Name the case before a GPU step runs, so a run that dies still says which one.
    if request.node.get_closest_marker("gpu") is not None:
        print(f"\n[case] {request.node.nodeid}", flush=True)
    yield
