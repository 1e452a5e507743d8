import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size case (minutes on the CPU oracle)")


def pytest_sessionfinish(session, exitstatus):
    """With QINT4_PARITY_REPORT=<path>, write every parity check's figures (relative L2
    of float32 outputs; largest relative error without the floor and the count of
    floor-rescued elements of bf16 outputs) as JSON."""
    path = os.environ.get("QINT4_PARITY_REPORT")
    if not path:
        return
    try:
        from tests import gpu_common
    except Exception:
        return
    import json

    with open(path, "w") as f:
        json.dump(gpu_common.REPORT, f, indent=0)
