import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workload (minutes of CPU oracle work)")


def pytest_collection_modifyitems(config, items):
    # GPU tests run only where a GPU is present; elsewhere they are skipped
    # rather than failing on import of the device runtime.
    try:
        import torch
        have_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        have_gpu = False
    if have_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU in this environment")
    for it in items:
        if "gpu" in it.keywords:
            it.add_marker(skip)


def pytest_sessionstart(session):
    import _support
    _support.tune_host_malloc()
    # MSA_TEST_LIB: run the tests on another build of the library (the
    # host-sanitized one: python -m nvfp4_kv_cache_amd.build --sanitize)
    lib = os.environ.get("MSA_TEST_LIB")
    if lib:
        import nvfp4_kv_cache_amd.binding as binding
        binding.LIB_PATH = lib
