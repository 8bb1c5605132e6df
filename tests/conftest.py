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
    """The CPU fp64 oracle, built from oracle/oracle.c if no build is present."""
    import oracle
    return oracle


@pytest.fixture(params=["auto", "nw8"])
def waves8(request, monkeypatch):
    """Workgroup shape: what the launch plan picks for the test's (small)
    grid, or eight query wavefronts (what large grids get; routed calls only
    with a four-head group, other head groups keep their shape)."""
    if request.param == "nw8":
        monkeypatch.setenv("ATTN_QUERY_WAVES", "8")
    return request.param
