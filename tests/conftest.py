import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def _gpu_available():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def pytest_collection_modifyitems(config, items):
    # GPU tests are selected with -m gpu; they fail loudly (not skip) when the
    # GPU or the library is missing, so a green GPU run always means native code ran.
    pass


@pytest.fixture(scope="session")
def lib():
    """The built C-ABI library, loaded through the Python binding."""
    import w4a16_int4_weight_linear_amd as w4
    return w4
