import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def oracle():
    import oracle as _oracle
    _oracle._load()
    return _oracle


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def osattn():
    """The HIP library's Python binding; GPU tests only."""
    if not gpu_available():
        pytest.skip("no GPU")
    import online_softmax_attention_amd as osa
    osa.load()  # raises if the built library is missing
    return osa
