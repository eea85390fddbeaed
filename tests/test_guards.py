"""The GPU tests' buffer guards (conftest._PoisoningTorch), exercised on host tensors: a buffer
cut out of a canary-filled allocation keeps its shape, dtype, contiguity and 16-byte alignment,
and a write one byte past either end of it is reported."""
import pytest
import torch

import conftest


@pytest.mark.parametrize("shape,dtype", [((3, 5, 7), torch.float32), ((4,), torch.uint8), ((2, 3), torch.bfloat16),
                                         ((0, 4), torch.float32), ((), torch.float32)])
def test_guarded_buffer_layout(shape, dtype):
    pt = conftest._PoisoningTorch(torch)
    x = pt._poison(pt._guarded(shape, dtype, "cpu"))
    raw, g = pt.guarded[-1]
    assert tuple(x.shape) == shape and x.dtype == dtype and x.is_contiguous()
    if x.numel():  # an empty view reports no data pointer
        assert x.data_ptr() - raw.data_ptr() == g and x.data_ptr() % 16 == 0
    if x.numel() and x.is_floating_point():
        assert torch.isnan(x.float()).all()


@pytest.mark.parametrize("where", ["head", "tail"])
def test_guard_overwrite_is_reported(where, monkeypatch):
    pt = conftest._PoisoningTorch(torch)
    monkeypatch.setattr(torch.cuda, "synchronize", lambda: None)
    pt._guarded((10,), torch.float32, "cpu").fill_(1.0)
    pt.check_guards()  # an in-bounds write leaves the guards intact
    pt._guarded((10,), torch.float32, "cpu")
    raw, g = pt.guarded[-1]
    raw[g - 1 if where == "head" else raw.numel() - g] = 0
    with pytest.raises(AssertionError, match="guard bytes"):
        pt.check_guards()
