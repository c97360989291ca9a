"""Shared pytest configuration: the ``gpu`` marker and the import path."""

import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


# KVQ_TEST_LIB: run the tests against another build of the library (the
# host-only sanitizer build of tests/test_host_sanitized.py)
if os.environ.get("KVQ_TEST_LIB"):
    from quantized_paged_kv_02_amd import kvq as _kvq
    _kvq.LIB = _kvq._load(os.environ["KVQ_TEST_LIB"], strict=False)
