import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def orc():
    """The CPU oracle (built on first use)."""
    from oracle import build as obuild
    from oracle import oracle as o
    if not os.path.exists(obuild.LIB):
        obuild.build()
    return o


@pytest.fixture(scope="session")
def mxq_lib():
    """The GPU library through its C ABI; fails loudly when it is not built."""
    from fp4_microscaling_quantization_amd import mxq
    return mxq
