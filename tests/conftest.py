import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: CPU test taking more than a few seconds")


@pytest.fixture
def hss_opt():
    """Setter for the library's diagnostic switches (hss_set_option), every
    switch it touched restored when the test ends."""
    import sparse_rank_linear_hss_amd as H
    saved = {}

    def set_(name, value):
        if name not in saved:
            saved[name] = H.hss_get_option(name)
        H.hss_set_option(name, value)

    yield set_
    for name, v in saved.items():
        H.hss_set_option(name, v)


def pytest_collection_modifyitems(config, items):
    # GPU tests cannot run without a device; make that a skip, not an error,
    # when someone runs the whole suite on a CPU-only machine.
    try:
        import torch
        have_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        have_gpu = False
    if have_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)
