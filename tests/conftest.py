import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs HIP kernels)")


@pytest.fixture(scope="session")
def oracle_lib():
    from oracle import oracle
    if not os.path.exists(oracle._LIB):
        oracle.build(force=False)
    return oracle


@pytest.fixture(scope="session")
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from paged_kv_cache_62_amd import pkv
    pkv.lib()  # raises if libpkv.so is missing: no fallback
    return torch.device("cuda:0")
