import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.dirname(os.path.abspath(__file__))
for p in (ROOT, HERE):
    if p not in sys.path:
        sys.path.insert(0, p)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


import pytest  # noqa: E402


@pytest.fixture(autouse=True)
def _clear_tuning_overrides():
    """Every test starts and ends with the library's default launch plans:
    tuning overrides (qoq_set_tuning) a test set are cleared afterwards."""
    yield
    import bit_integer_gemm_amd as qoq
    if qoq._LIB is not None:
        qoq.clear_tuning()
