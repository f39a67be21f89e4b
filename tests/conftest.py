import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def _may_run_gpu_tests(config) -> bool:
    return (config.getoption("-m") or "").strip() != "not gpu"


def pytest_sessionstart(session):
    # The full-size parity checks run the oracle in forked workers. Fork them
    # now, before collection asks whether a GPU is there (which initialises
    # it), so no worker inherits an initialised device.
    if _may_run_gpu_tests(session.config):
        from tests import _oracle_pool

        _oracle_pool.start()


def pytest_sessionfinish(session, exitstatus):
    from tests import _oracle_pool

    _oracle_pool.stop()


def _gpu_available():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def pytest_collection_modifyitems(config, items):
    if _gpu_available():
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for it in items:
        if "gpu" in it.keywords:
            it.add_marker(skip)
