import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs the HIP kernels)")


@pytest.fixture(scope="session")
def oracle_lib():
    """The CPU oracle, built with gcc if it has not been built yet."""
    import oracle
    if not os.path.exists(oracle.LIBRARY):
        oracle.build()
    return oracle


@pytest.fixture(scope="session")
def pa():
    """The HIP library's binding; builds libpa.so only if it is missing."""
    import paged_kv_cache_05_amd as pa_mod
    if not os.path.exists(pa_mod.LIBRARY):
        from paged_kv_cache_05_amd import _build
        _build.build()
    pa_mod.library()
    return pa_mod


@pytest.fixture(scope="session")
def device(pa):
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a visible GPU")
    return torch.device("cuda:0")
