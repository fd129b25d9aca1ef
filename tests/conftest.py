import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: takes more than a few seconds")


@pytest.fixture(scope="session")
def oracle_mod():
    import oracle

    oracle.build()
    return oracle


@pytest.fixture(scope="session")
def hata_gpu():
    """The HIP library binding on cuda:0 (GPU tests only)."""
    import torch

    if not torch.cuda.is_available():
        pytest.fail("GPU test collected without a GPU")
    from hash_top_sparse_amd import binding

    binding.load()
    return binding
