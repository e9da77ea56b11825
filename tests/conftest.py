import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: large CPU-side work (full-size oracle runs)")


def pytest_collection_modifyitems(config, items):
    # keep GPU tests from running (and failing) where no GPU is visible, but only
    # when the caller did not ask for them explicitly with -m gpu
    markexpr = config.getoption("-m") or ""
    if "gpu" in markexpr and "not gpu" not in markexpr:
        return
    try:
        import torch
        has_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        has_gpu = False
    if has_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for it in items:
        if "gpu" in it.keywords:
            it.add_marker(skip)


@pytest.fixture(scope="session")
def qmvlib():
    """The built C-ABI library (built in-tree first if nothing is built yet)."""
    from quantized_matvec_amd import build, qmv
    if not os.path.exists(qmv.library_path):
        build.build()
    return qmv.lib()
