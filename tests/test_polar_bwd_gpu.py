"""GPU parity of the Polar attention backward (atma_polar_attn_fwd_train + atma_polar_attn_bwd)
against the fp64 oracle's gradients (``oracle.polar_bwd``, pinned by finite differences).

Every element of dq, dk, dv and of the parameter gradients is compared on the same seeded bf16
inputs and a seeded bf16 upstream gradient, by two measures: max |gpu - oracle| / max |oracle|
<= 2e-2 (each tensor against its own scale) and ||gpu - oracle||_F / ||oracle||_F <= 1e-2.  The
four scalar parameter gradients are sums over every row whose terms cancel; each is judged
against the sum of its rows' magnitudes (returned by the oracle), <= 2e-2.

Why not the forward's max |error| / rms: the gradients are heavy-tailed (the largest elements are
10-20 times the RMS) and each element is a sum over keys or queries whose terms are set by the
largest products of its row, so bf16 arithmetic leaves an absolute error proportional to the
tensor's top scale.  The backward contracts on bf16 MFMA with three intermediates rounded to bf16
in series (the direction-sum gradient ds, the weights for dV, the logit gradient for dq and dk,
each to 2^-9 relative) on top of the forward's own bf16-level direction and magnitude; measured on
these cases that gives a Frobenius error of about 3e-3 (1.5 x 2^-9) and a max error of 4-6e-3 of
the top scale -- but 4-12e-2 of the RMS, growing with T as the tails do.  The budgets above leave a
factor three; a missing or wrong term moves either measure by O(1).
Cases span several
128-query / 128-key tiles with ragged tails, one and several query heads per kv head, head
widths 64 and 128, a single-token sequence, and the clamped direction normaliser.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import (POLAR_BWD_TOL_FRO as TOL_FRO, POLAR_BWD_TOL_MAX as TOL_MAX, POLAR_GRADS, note,
                    polar_grad_errors, polar_grad_failures, rel_err_fro, rel_err_max, to_np)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def atma():
    import gated_delta_memory_amd as g

    assert torch.cuda.is_available()
    return g


def _run(atma, inp, do, eps=None):
    p = {k: (v.cuda() if torch.is_tensor(v) else v) for k, v in inp["params"].items()}
    if eps is not None:
        p["eps"] = eps
    q, k, v = (inp[x].cuda() for x in ("q", "k", "v"))
    o, mu, stats, dirn = atma.atma_polar_attn_fwd_train(q, k, v, p)
    g = atma.atma_polar_attn_bwd(q, k, v, p, mu, stats, dirn, do.cuda())
    torch.cuda.synchronize()
    return o, mu, g


def _case(B, T, Hq, Hkv, D, seed):
    inp = workloads.make_polar_inputs(B, T, Hq, Hkv, D, seed=seed)
    gen = torch.Generator().manual_seed(seed + 1)
    do = torch.randn(B, T, Hq, D, generator=gen).to(torch.bfloat16)
    return inp, do


def _check(atma, B, T, Hq, Hkv, D, seed, eps=None):
    inp, do = _case(B, T, Hq, Hkv, D, seed)
    o, mu, g = _run(atma, inp, do, eps)
    cp = {k: (v.cpu() if torch.is_tensor(v) else v) for k, v in inp["params"].items()}
    if eps is not None:
        cp["eps"] = eps
    ref = oracle.polar_bwd(inp["q"], inp["k"], inp["v"], cp, do)
    errs = polar_grad_errors({n: to_np(g[n]) for n in POLAR_GRADS}, ref)
    note(f"  polar bwd B{B} T{T} Hq{Hq} Hkv{Hkv} D{D}: " +
         " ".join(f"{n}={e[0]:.1e}/{e[1]:.1e}" for n, e in errs.items()))
    bad = polar_grad_failures(errs)
    assert not bad, bad
    return o, mu


@pytest.mark.parametrize("B,T,Hq,Hkv,D", [(1, 1, 1, 1, 64), (1, 77, 2, 2, 64), (2, 300, 4, 2, 64),
                                          (1, 513, 3, 1, 64), (2, 256, 2, 2, 64), (1, 200, 8, 2, 128),
                                          (1, 640, 2, 2, 128), (2, 129, 4, 4, 128), (1, 2048, 4, 2, 64),
                                          (1, 1024, 8, 2, 128)])
def test_polar_bwd_matches_oracle(atma, B, T, Hq, Hkv, D):
    _check(atma, B, T, Hq, Hkv, D, seed=1000 + T + Hq + D)


@pytest.mark.parametrize("T", [63, 64, 65, 127, 128, 129])
def test_polar_bwd_tile_edges(atma, T):
    """Lengths at and around the 64-row streamed blocks and the 128-row tiles (padding rows of
    the row-scalar layout, ragged last key and query blocks)."""
    _check(atma, 1, T, 2, 1, 64, seed=4000 + T)


def test_polar_bwd_needle_keys(atma):
    """Peaked attention: 10% of the keys are repeated needles (the 16K workload's key mixture), so
    many rows put most of their weight on a few keys and the gradients are strongly heavy-tailed."""
    inp = workloads.make_polar_inputs(1, 400, 4, 2, 64, seed=61, needle_frac=0.1)
    gen = torch.Generator().manual_seed(62)
    do = torch.randn(1, 400, 4, 64, generator=gen).to(torch.bfloat16)
    _, _, g = _run(atma, inp, do)
    cp = {k: (v.cpu() if torch.is_tensor(v) else v) for k, v in inp["params"].items()}
    ref = oracle.polar_bwd(inp["q"], inp["k"], inp["v"], cp, do)
    errs = polar_grad_errors({n: to_np(g[n]) for n in POLAR_GRADS}, ref)
    note("  polar bwd needles: " + " ".join(f"{n}={e[0]:.1e}/{e[1]:.1e}" for n, e in errs.items()))
    bad = polar_grad_failures(errs)
    assert not bad, bad


def test_polar_bwd_clamped_normaliser(atma):
    """eps above every ||s||: the direction gradient has no projection term."""
    _check(atma, 1, 150, 2, 1, 64, seed=77, eps=30.0)


def test_polar_train_forward_matches_inference_forward(atma):
    """The training forward writes the same o and mu as the inference forward (bitwise), a unit
    direction whose scaling by mu is o, and row statistics consistent with m_eff = R^3 / Q2."""
    inp = workloads.make_polar_inputs(2, 333, 4, 2, 64, seed=5)
    p = {k: (v.cuda() if torch.is_tensor(v) else v) for k, v in inp["params"].items()}
    q, k, v = (inp[x].cuda() for x in ("q", "k", "v"))
    o1, mu1, meff1 = atma.atma_polar_attn_fwd(q, k, v, p, want_mu=True)
    o2, mu2, stats, dirn = atma.atma_polar_attn_fwd_train(q, k, v, p)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(mu1, mu2)
    d = to_np(dirn)
    np.testing.assert_allclose(np.linalg.norm(d, axis=-1), 1.0, rtol=1e-5)
    np.testing.assert_allclose(d * to_np(mu2).transpose(0, 2, 1)[..., None], to_np(o2), atol=8e-3)
    st = to_np(stats)
    np.testing.assert_allclose(st[..., 1] ** 3 / st[..., 2], to_np(meff1), rtol=1e-4)
    assert np.all(st[..., 1] > 0) and np.all(st[..., 1] <= 1 + 1e-6) and np.all(st[..., 3] > 0)


def test_polar_bwd_is_deterministic(atma):
    inp, do = _case(2, 300, 4, 2, 64, seed=9)
    _, _, g1 = _run(atma, inp, do)
    _, _, g2 = _run(atma, inp, do)
    for n in g1:
        assert torch.equal(g1[n], g2[n]), n


def test_polar_bwd_layer_b8_t2k(atma):
    """The 2K layer as the benchmark times it (B=8, T=2048, Hq=Hkv=16, D=64, one launch over the
    whole batch); the oracle's gradients of batch 0 (the kernels treat every batch the same)."""
    inp = workloads.make_workload("layer_b8_t2k")["polar"]
    B, T, Hq, D = inp["q"].shape
    do = torch.randn(B, T, Hq, D, generator=torch.Generator().manual_seed(2048)).to(torch.bfloat16)
    _, _, g = _run(atma, inp, do)
    cp = {k: (v.cpu() if torch.is_tensor(v) else v) for k, v in inp["params"].items()}
    ref = oracle.polar_bwd(inp["q"][:1], inp["k"][:1], inp["v"][:1], cp, do[:1])
    for n in ("dq", "dk", "dv"):
        em, ef = rel_err_max(to_np(g[n])[:1], ref[n]), rel_err_fro(to_np(g[n])[:1], ref[n])
        note(f"  polar bwd layer_b8_t2k batch 0 {n}: {em:.1e}/{ef:.1e}")
        assert em <= TOL_MAX and ef <= TOL_FRO, (n, em, ef)
