import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")


@pytest.fixture(scope="session")
def golden_dir():
    return os.path.join(ROOT, "tests", "golden")


@pytest.fixture(autouse=True)
def _automatic_dispatch():
    """Every test starts and ends with the library's automatic dispatch
    choices (tests force tiles and paths through qg.set_override)."""
    yield
    from weight_only_quantized_w8a16_amd import _abi
    if _abi._lib is not None:
        import weight_only_quantized_w8a16_amd as qg
        qg.clear_override()
