import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


import pytest


@pytest.fixture
def force_plan():
    """force_plan(family, kind, splits=0): nvfp4_force_plan for the rest of
    the test; every family is back to the library's own choice afterwards."""
    import nvfp4_block_scaled_07_amd as nv

    def force(family, kind, splits=0):
        nv.nvfp4_force_plan(family, kind, splits)
    yield force
    for fam in (nv.FAMILY_GEMM, nv.FAMILY_MX, nv.FAMILY_GROUPED):
        nv.nvfp4_force_plan(fam, -1, 0)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
