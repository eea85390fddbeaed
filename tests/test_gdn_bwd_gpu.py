"""GPU parity of the memory backward (atma_gdn_bwd) against the fp64 oracle's gradients
(``oracle.gdn_bwd``, the reverse pass over the token recurrence, pinned by finite differences).

Every element of dq, dk, dv, dalpha, dbeta and of the initial-state gradient is compared on the
same seeded inputs (unit-norm q and k, as the forward assumes), a seeded upstream gradient on the
outputs and, in some cases, on the final state.  The kernels compute in fp32 throughout (inputs
converted exactly), so the budgets are those of fp32 arithmetic over a few hundred chunked
products: max |gpu - oracle| / max |oracle| <= 1e-4 for fp32 inputs; for bf16 inputs the
outputs dq, dk, dv are stored in bf16 (their own rounding, 2^-9 of an element, is at most
2^-9 of the tensor's top scale), so 4e-3 there and 1e-4 for the fp32 outputs dalpha, dbeta and
the state gradient.  Frobenius errors are reported beside.  Cases cover ragged last chunks,
every (Dk, Dv) pair, an initial state and an upstream gradient on the final state, one token,
and a sequence of 16 chunks.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import GDN_GRADS, gdn_grad_errors, gdn_grad_failures, note, rel_err_fro, rel_err_max, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def atma():
    import gated_delta_memory_amd as g

    assert torch.cuda.is_available()
    return g


def _check(atma, B, T, H, Dk, Dv, dtype, init, final, seed):
    inp = workloads.make_gdn_inputs(B, T, H, Dk, Dv, dtype=dtype, seed=seed)
    gen = torch.Generator().manual_seed(seed + 7)
    td = workloads.torch_dtype(dtype)
    do = torch.randn(B, T, H, Dv, generator=gen).to(td)
    S0 = torch.randn(B, H, Dv, Dk, generator=gen) * 0.3 if init else None
    dSf = torch.randn(B, H, Dv, Dk, generator=gen) * 0.5 if final else None
    cu = lambda x: None if x is None else x.cuda()  # noqa: E731
    g = atma.atma_gdn_bwd(cu(inp["q"]), cu(inp["k"]), cu(inp["v"]), cu(inp["alpha"]), cu(inp["beta"]), cu(do),
                          init_state=cu(S0), dS_final=cu(dSf), want_dinit=True)
    torch.cuda.synchronize()
    ref = oracle.gdn_bwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], do, init_state=S0, dS_final=dSf)
    errs = gdn_grad_errors({n: to_np(g[n]) for n in GDN_GRADS}, ref)
    note(f"  gdn bwd B{B} T{T} H{H} Dk{Dk} Dv{Dv} {dtype}: " +
         " ".join(f"{n}={e[0]:.1e}/{e[1]:.1e}" for n, e in errs.items()))
    bad = gdn_grad_failures(errs, dtype)
    assert not bad, bad


@pytest.mark.parametrize("B,T,H,Dk,Dv,dtype,init,final", [
    (1, 1, 1, 64, 64, "bf16", False, False),
    (1, 77, 2, 64, 64, "bf16", True, True),
    (2, 200, 2, 128, 128, "bf16", False, False),
    (1, 130, 3, 64, 128, "f32", True, False),
    (1, 300, 1, 128, 64, "f32", False, True),
    (2, 64, 2, 128, 128, "bf16", True, True),
    (1, 1000, 1, 128, 128, "bf16", True, True),
    (1, 257, 2, 128, 128, "f32", True, True),
])
def test_gdn_bwd_matches_oracle(atma, B, T, H, Dk, Dv, dtype, init, final):
    _check(atma, B, T, H, Dk, Dv, dtype, init, final, seed=100 + T + Dk + Dv)


@pytest.mark.parametrize("T", [63, 64, 65, 128, 129])
def test_gdn_bwd_chunk_edges(atma, T):
    """Lengths at and around the 64-token chunk (a ragged last chunk of 1 and of 63 tokens)."""
    _check(atma, 1, T, 2, 64, 128, "bf16", True, True, seed=300 + T)


def test_gdn_bwd_is_deterministic(atma):
    inp = workloads.make_gdn_inputs(1, 150, 2, 128, 128, seed=3)
    do = torch.randn(1, 150, 2, 128, generator=torch.Generator().manual_seed(4)).to(torch.bfloat16)
    args = [inp[x].cuda() for x in ("q", "k", "v", "alpha", "beta")] + [do.cuda()]
    g1 = atma.atma_gdn_bwd(*args, want_dinit=True)
    g2 = atma.atma_gdn_bwd(*args, want_dinit=True)
    torch.cuda.synchronize()
    for n in g1:
        assert torch.equal(g1[n], g2[n]), n


def test_gdn_bwd_layer_b8_t2k(atma):
    """The 2K layer as the benchmark times it (B=8, T=2048, H=8, d=128, bf16, one launch over the
    whole batch); the oracle's gradients of batch 0 (the kernels treat every batch the same)."""
    inp = workloads.make_workload("layer_b8_t2k")["gdn"]
    B, T, H, D = inp["q"].shape
    do = torch.randn(B, T, H, D, generator=torch.Generator().manual_seed(2049)).to(torch.bfloat16)
    g = atma.atma_gdn_bwd(*[inp[x].cuda() for x in ("q", "k", "v", "alpha", "beta")], do.cuda(), want_dinit=True)
    torch.cuda.synchronize()
    ref = oracle.gdn_bwd(inp["q"][:1], inp["k"][:1], inp["v"][:1], inp["alpha"][:1], inp["beta"][:1], do[:1])
    for n in ("dq", "dk", "dv", "dalpha", "dbeta", "dinit"):
        em, ef = rel_err_max(to_np(g[n])[:1], ref[n]), rel_err_fro(to_np(g[n])[:1], ref[n])
        note(f"  gdn bwd layer_b8_t2k batch 0 {n}: {em:.1e}/{ef:.1e}")
        tol = 4e-3 if n in ("dq", "dk", "dv") else 1e-4
        assert em <= tol and ef <= tol, (n, em, ef)
