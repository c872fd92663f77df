import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD GPU (MI355X / gfx950) and the built HIP library")


@pytest.fixture
def forcer():
    """forcer(path=..., gemm=..., decode=..., pair=...): force kernels for the rest of the test (the library's
    test-only hook, per thread); the automatic choice is restored at teardown."""
    stack = []

    def force(**kw):
        from bit_weight_linear_amd import binding as B
        cm = B.forced_kernels(**kw)
        cm.__enter__()
        stack.append(cm)

    yield force
    while stack:
        stack.pop().__exit__(None, None, None)
