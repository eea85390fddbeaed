import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def rng():
    import numpy as np

    return np.random.default_rng(1234)


class _PoisoningTorch:
    """Stands in for ``torch`` inside the binding during GPU tests: every buffer the binding
    allocates (outputs, workspaces) comes back filled with NaN (floating dtypes) or 0xFF bytes
    (a byte workspace: read as fp32, fp16 or bf16 that is NaN too), never with the stale contents
    of an earlier call, so an element a kernel fails to write cannot pass on leftovers."""

    def __init__(self, torch):
        self._t = torch

    def __getattr__(self, name):
        return getattr(self._t, name)

    def _poison(self, x):
        if x.is_floating_point():
            return x.fill_(float("nan"))
        if x.dtype == self._t.uint8:
            return x.fill_(0xFF)
        return x

    def empty(self, *a, **k):
        return self._poison(self._t.empty(*a, **k))

    def empty_like(self, *a, **k):
        return self._poison(self._t.empty_like(*a, **k))


@pytest.fixture(autouse=True)
def poison_binding_buffers(request, monkeypatch):
    if request.node.get_closest_marker("gpu") is None:
        yield
        return
    import torch

    import gated_delta_memory_amd as g

    monkeypatch.setattr(g, "torch", _PoisoningTorch(torch))
    yield
