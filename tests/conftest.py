import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")
    # The every-row parity tests evaluate the oracle in worker processes
    # forked from a forkserver; it must start before anything initialises the
    # GPU (counting devices does not).
    try:
        import torch
        if torch.cuda.device_count() > 0:
            from tests import oracle_pool
            oracle_pool.start()
    except Exception:
        pass


def pytest_collection_modifyitems(config, items):
    # GPU tests are skipped, not failed, where there is no GPU; the product
    # path itself still fails loudly when its library is missing.
    try:
        import torch
        have_gpu = torch.cuda.is_available()
    except Exception:
        have_gpu = False
    if have_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)
