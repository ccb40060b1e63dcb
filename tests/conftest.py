import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_collection_modifyitems(config, items):
    # With an explicit -m expression pytest itself selects or deselects the GPU tests;
    # a GPU test selected with -m gpu then fails loudly when there is no GPU. Only an
    # unfiltered run on a machine without a GPU skips them here.
    if config.getoption("-m"):
        return
    if not any("gpu" in item.keywords for item in items):
        return
    import torch
    if torch.cuda.is_available():
        return
    skip = pytest.mark.skip(reason="no GPU in this process; run with -m gpu on an MI355X")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)
