import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# HYS_TEST_LIB: run the CPU tests against another build of the library (the
# host-checked build of tests/test_checked_build.py); such a run has no GPU
CHECKED_RUN = bool(os.environ.get("HYS_TEST_LIB"))
if CHECKED_RUN:
    from hybrid_sparse_attention_flash_amd import _lib as _hys_lib
    _hys_lib.load(os.environ["HYS_TEST_LIB"])


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU oracle case")


def pytest_collection_modifyitems(config, items):
    # GPU tests are skipped automatically when no GPU is visible, so that
    # `-m "not gpu"` and a plain run on a CPU host both stay green.
    has_gpu = False
    if not CHECKED_RUN:
        try:
            import torch
            has_gpu = torch.cuda.is_available()
        except Exception:
            has_gpu = False
    if has_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for it in items:
        if "gpu" in it.keywords:
            it.add_marker(skip)
