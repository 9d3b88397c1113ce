import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: full-size inputs; minutes on the CPU")


@pytest.fixture(scope="session")
def dev():
    """cuda:0 with the library loaded (a GPU test fails loudly if it is not
    built; there is no fallback)."""
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_paged_kv_03_amd as lib
    lib._lib.lib()
    return torch.device("cuda:0")
