import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

POISON = 0xA5


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


@pytest.fixture(scope="session")
def orc():
    import oracle
    oracle.lib()
    return oracle


@pytest.fixture(autouse=True)
def poisoned_outputs(request, monkeypatch):
    """In GPU tests every output the binding allocates starts as 0xA5 bytes, so an element a kernel
    fails to write cannot pass by holding the expected value from an earlier allocation."""
    if request.node.get_closest_marker("gpu") is None:
        yield
        return
    import torch
    from precision_rl_amd import fp4q

    def alloc(shape, dtype, device):
        t = torch.empty(shape, dtype=dtype, device=device)
        t.view(torch.uint8).fill_(POISON)
        return t
    monkeypatch.setattr(fp4q, "_alloc", alloc)
    yield
