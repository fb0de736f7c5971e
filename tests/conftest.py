import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs through the HIP C-ABI)")
    config.addinivalue_line(
        "markers", "oracle_full(job): compares with a background oracle job of tests/oracle_pool.py"
    )


def _gpu_available():
    try:
        import torch

        return torch.cuda.is_available()
    except Exception:
        return False


def pytest_collection_modifyitems(config, items):
    if _gpu_available():
        return
    skip = pytest.mark.skip(reason="no GPU in this environment")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


def pytest_collection_finish(session):
    """Start the background oracle jobs of the selected full-size parity
    tests (worker processes that never touch the GPU), so that they run while
    the other GPU tests do."""
    jobs = []
    for item in session.items:
        if item.get_closest_marker("skip"):
            continue
        m = item.get_closest_marker("oracle_full")
        if m:
            jobs.extend(a for a in m.args if a not in jobs)
    if jobs and _gpu_available():
        import oracle_pool

        oracle_pool.start(jobs)


def pytest_sessionfinish(session, exitstatus):
    mod = sys.modules.get("oracle_pool")
    if mod is not None:
        mod.shutdown()
