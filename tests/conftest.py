import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")
    # The GPU parity tests run the oracle on CPU worker processes.  Their fork
    # server starts here, before anything in this process touches the GPU, so
    # no worker is ever forked from (or execs out of) a process holding it.
    if "not gpu" not in (config.getoption("markexpr", "") or ""):
        from tests.oracle_pool import start_server
        start_server()


def pytest_collection_modifyitems(config, items):
    # GPU tests run only where a GPU is visible; on a GPU machine they never
    # skip silently: a missing library fails them loudly.
    try:
        import torch
        has_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        has_gpu = False
    if has_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)
