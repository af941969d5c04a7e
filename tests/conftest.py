import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def golden_path(name):
    return os.path.join(GOLDEN, name)


def read_golden(name):
    """Non-comment, non-blank lines of a golden text fixture."""
    with open(golden_path(name)) as f:
        return [ln.strip() for ln in f if ln.strip() and not ln.lstrip().startswith("#")]


@pytest.fixture(scope="session")
def golden():
    return read_golden


def pytest_collection_modifyitems(config, items):
    """GPU tests are skipped, with a reason, on a machine without a GPU."""
    if not any("gpu" in it.keywords for it in items):
        return
    import torch
    if torch.cuda.is_available():
        return
    skip = pytest.mark.skip(reason="no GPU visible to torch")
    for it in items:
        if "gpu" in it.keywords:
            it.add_marker(skip)
