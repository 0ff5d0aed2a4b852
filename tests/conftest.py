import os
import sys

import numpy as np
import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


from oracle.adapters import appended_pools, oracle_args, prefill_args, \
    raw, raw_bits  # noqa: E402,F401


@pytest.fixture(scope="session")
def gpu_lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from paged_kv_cache_451_amd import _lib
    return _lib.load()
