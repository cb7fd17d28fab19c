import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def _redirect_libraries():
    """GDN_TEST_LIBGDN / GDN_TEST_ORACLE: run the tests against other builds of the two libraries
    (the AddressSanitizer builds of tests/test_host_asan.py)."""
    lib, orc = os.environ.get("GDN_TEST_LIBGDN"), os.environ.get("GDN_TEST_ORACLE")
    if lib:
        import linear_attention_sequence_rule_amd as gdn
        gdn._LIB_PATH = lib
    if orc:
        import oracle
        oracle._LIB = orc
        oracle.build = lambda force=True: orc


_redirect_libraries()


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD Instinct GPU (gfx950) and libgdn.so")
    config.addinivalue_line("markers", "slow: long-running (full-size) case")


def _has_gpu():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:  # pragma: no cover
        return False


def pytest_collection_modifyitems(config, items):
    if _has_gpu():
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)
