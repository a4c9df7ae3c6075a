import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


import pytest  # noqa: E402


@pytest.fixture(params=["long_double", "fp64"])
def orc(request):
    """Both builds of the CPU oracle: the long double reference and the fp64
    variant timed as the CPU baseline; every pin holds for both."""
    import oracle

    return oracle.default() if request.param == "long_double" else oracle.fp64()
