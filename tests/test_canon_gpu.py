"""GPU parity of the Canon prologue (depthwise causal convolution, residual, per-head unit
norm, carried state) against the fp64 oracle.  Output is bf16: the budget is 2e-2 of the RMS
beyond one bf16 ulp, as for every bf16 output."""
import numpy as np
import pytest
import torch

import oracle
from parity import TOL, note, out_err, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def atma():
    import gated_delta_memory_amd as g

    assert torch.cuda.is_available()
    return g


def _inputs(B, T, C, K, seed, with_state):
    gen = torch.Generator().manual_seed(seed)
    x = torch.randn(B, T, C, generator=gen).to(torch.bfloat16)
    w = torch.randn(K, C, generator=gen) * 0.5
    st = torch.randn(B, K - 1, C, generator=gen).to(torch.bfloat16) if with_state and K > 1 else None
    return x, w, st


@pytest.mark.parametrize("B,T,C,K,res,heads,st", [(1, 1, 8, 1, 0, 0, False), (2, 300, 1024, 4, 1, 8, True),
                                                  (3, 77, 256, 3, 0, 4, False), (1, 2048, 1024, 4, 1, 0, True),
                                                  (2, 5, 512, 8, 1, 16, True), (1, 100, 64, 2, 0, 1, False)])
def test_canon_matches_oracle(atma, B, T, C, K, res, heads, st):
    x, w, state = _inputs(B, T, C, K, T + C + K, st)
    sd = None if state is None else state.cuda().clone()
    y = atma.atma_canon(x.cuda(), w.cuda(), sd, residual=bool(res), heads=heads)
    torch.cuda.synchronize()
    ref = oracle.canon(x, w, state=state, residual=bool(res), heads=heads)
    e = out_err(to_np(y), ref, "bf16")
    note(f"  canon B{B} T{T} C{C} K{K} res{res} heads{heads} state{st} err={e:.3e}")
    assert e <= TOL["bf16"]
    if sd is not None:  # the new state holds the last K-1 inputs (exact copies)
        full = torch.cat([state, x], dim=1)
        assert torch.equal(sd.cpu(), full[:, -(K - 1):])


def test_canon_decode_steps_equal_prefill(atma):
    """Token-by-token calls with the state updated in place give the prefill result."""
    B, T, C, K = 2, 40, 1024, 4
    x, w, _ = _inputs(B, T, C, K, 7, False)
    xd, wd = x.cuda(), w.cuda()
    y = atma.atma_canon(xd, wd, None, residual=True, heads=8)
    state = torch.zeros(B, K - 1, C, dtype=torch.bfloat16, device="cuda")
    steps = [atma.atma_canon(xd[:, t:t + 1].contiguous(), wd, state, residual=True, heads=8) for t in range(T)]
    torch.cuda.synchronize()
    assert torch.equal(torch.cat(steps, dim=1), y)
