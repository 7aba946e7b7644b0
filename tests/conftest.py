import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built libfa")


@pytest.fixture(autouse=True)
def _parity_test_id(request):
    """Tag the parity records of the running test with its id."""
    gu = sys.modules.get("gpu_util")
    if gu is not None:
        gu.CURRENT_TEST["id"] = request.node.nodeid
    yield


def pytest_sessionfinish(session, exitstatus):
    """With FA_PARITY_REPORT=<path>, write every parity comparison of the session
    to <path> (JSON) and a per-workload table to <path>.md."""
    path = os.environ.get("FA_PARITY_REPORT")
    gu = sys.modules.get("gpu_util")
    if path and gu is not None and gu.RECORDS:
        gu.write_report(path)
