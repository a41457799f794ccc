import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")


@pytest.fixture(scope="session")
def kvc():
    """The HIP library's binding; a GPU test fails loudly if it is not built."""
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import kv_cache_attention_kvcache_amd as m  # raises ImportError when libkvc.so is missing

    return m
