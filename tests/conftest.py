import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    # The sanitizer tier (test_sanitizers.py) runs the host-side ABI tests
    # against a host-only build of the library's host layer made with
    # AddressSanitizer and UndefinedBehaviorSanitizer: it names that build here.
    host_lib = os.environ.get("KDA_TEST_HOST_LIBRARY")
    if host_lib:
        import linear_attention_recurrent_decode_amd as kda
        kda._lib = kda._open(host_lib)


def pytest_collection_modifyitems(config, items):
    # GPU tests skip only where no GPU exists at all; on a GPU machine they
    # run and fail loudly if the HIP library is missing.
    try:
        import torch
        have_gpu = torch.cuda.is_available()
    except Exception:
        have_gpu = False
    if have_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU in this machine")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)
