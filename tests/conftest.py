import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_collection_modifyitems(config, items):
    # GPU tests are only meaningful where a GPU is visible; elsewhere they are skipped
    # (on a GPU machine they are selected with -m gpu).
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


def pytest_runtest_setup(item):
    # Name each GPU case on stderr (unbuffered) before it runs, so a failing or hanging
    # GPU step can be attributed from the tail of the output.
    if "gpu" in item.keywords:
        sys.stderr.write("\n[gpu-case] %s\n" % item.nodeid)
        sys.stderr.flush()
