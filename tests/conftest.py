import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")


def golden_path(name: str) -> str:
    return os.path.join(ROOT, "tests", "golden", name)


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP library, loaded once; skips nothing: a GPU test without it fails loudly."""
    import torch

    if not torch.cuda.is_available():
        pytest.fail("gpu test selected but no GPU is visible")
    from sparse_attention_13_amd import binding

    binding.load()  # raises when the extension is missing
    return binding
