import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# every test layer fills its workspace with 0xFF bytes before each eager
# route, permute and forward: a kernel that reads workspace memory no
# earlier kernel of the same call wrote then gives wrong results
os.environ.setdefault("MOE_POISON_WORKSPACE", "1")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: large-shape case (seconds to minutes)")


def pytest_collection_modifyitems(config, items):
    # GPU tests are skipped (not failed) where no GPU is visible, so that
    # `-m "not gpu"` and plain runs both work on a CPU-only machine.
    try:
        import torch
        have_gpu = torch.cuda.is_available()
    except Exception:
        have_gpu = False
    if have_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for it in items:
        if "gpu" in it.keywords:
            it.add_marker(skip)
