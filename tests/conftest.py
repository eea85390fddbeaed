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


GUARD_BYTES = 4096  # keeps the 16-byte (and 512-byte) alignment of the allocator's blocks
CANARY = 0xA5


class _PoisoningTorch:
    """Stands in for ``torch`` inside the binding during GPU tests: every buffer the binding
    allocates (outputs, workspaces) comes back filled with NaN (floating dtypes) or 0xFF bytes
    (a byte workspace: read as fp32, fp16 or bf16 that is NaN too), never with the stale contents
    of an earlier call, so an element a kernel fails to write cannot pass on leftovers.  Device
    buffers are also cut out of a larger allocation with GUARD_BYTES of canary bytes on each side;
    after the test every guard band must still hold the canary, so a kernel that writes past
    either end of a buffer it was given fails the test that ran it."""

    def __init__(self, torch):
        self._t = torch
        self.guarded = []  # (flat uint8 view of the whole allocation, guard bytes)

    def __getattr__(self, name):
        return getattr(self._t, name)

    def _poison(self, x):
        if x.is_floating_point():
            return x.fill_(float("nan"))
        if x.dtype == self._t.uint8:
            return x.fill_(0xFF)
        return x

    def _guarded(self, shape, dtype, device):
        t = self._t
        n = 1
        for d in shape:
            n *= int(d)
        es = t.empty((), dtype=dtype).element_size()
        g = GUARD_BYTES // es
        raw = t.empty((n + 2 * g) * es, dtype=t.uint8, device=device)
        raw.fill_(CANARY)
        self.guarded.append((raw, GUARD_BYTES))
        return raw.view(dtype)[g:g + n].view(tuple(shape))

    def empty(self, *a, **k):
        shape = a[0] if len(a) == 1 and isinstance(a[0], (tuple, list, self._t.Size)) else a
        dev = k.get("device")
        if dev is not None and self._t.device(dev).type == "cuda" and not k.get("pin_memory", False):
            dtype = k.get("dtype") or self._t.get_default_dtype()
            return self._poison(self._guarded(tuple(shape), dtype, dev))
        return self._poison(self._t.empty(*a, **k))

    def empty_like(self, x, **k):
        if x.is_cuda and not k:
            return self._poison(self._guarded(tuple(x.shape), x.dtype, x.device))
        return self._poison(self._t.empty_like(x, **k))

    def check_guards(self):
        self._t.cuda.synchronize()
        for raw, g in self.guarded:
            head, tail = raw[:g], raw[raw.numel() - g:]
            bad = int((head != CANARY).sum().item()) + int((tail != CANARY).sum().item())
            assert bad == 0, f"{bad} guard bytes around a {raw.numel() - 2 * g}-byte buffer were overwritten"
        self.guarded.clear()


@pytest.fixture(autouse=True)
def poison_binding_buffers(request, monkeypatch):
    if request.node.get_closest_marker("gpu") is None:
        yield
        return
    import torch

    import gated_delta_memory_amd as g

    pt = _PoisoningTorch(torch)
    monkeypatch.setattr(g, "torch", pt)
    yield
    pt.check_guards()
