"""GPU parity of the NoPE / RoPE control cores (causal softmax attention, rotary embedding)
against the fp64 oracle.  Budget: 2e-2 beyond the output cast (u = 2^-8), per output row against the row's
own RMS (plain softmax rows shrink ~1/sqrt(keys seen); see parity.rel_err_rows_bf16).

RoPE prefill is compared with the EXACT rotation.  The kernel consumes the rotated q and k as
bf16 MFMA operands, which moves the output by an amount the oracle states per element: the
probabilistic rounding tolerance of ``oracle.softmax_attn(..., tol_lambda=7)`` (Hoeffding bound
on the first-order effect of independent roundings of relative size <= 2^-8, 7 standard
deviations).  That tolerance is allowed on top of the usual budget.  A second check compares
with the composition the library performs (atma_rope's bf16 output, oracle.rope(bf16=True),
then the NoPE core) at the plain budget.  RoPE decode reads a cache of keys already rotated to
their slots (a RoPE KV cache holds them so), built here by the oracle's rope with bf16 output;
the query is rotated inside the kernel in fp32, so decode is compared with no extra allowance."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import TOL, note, out_err, rel_err_rows_bf16, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def atma():
    import gated_delta_memory_amd as g

    assert torch.cuda.is_available()
    return g


@pytest.mark.parametrize("pos0", [0, 262000])
def test_rope_matches_oracle(atma, pos0):
    """Positions up to 262300: the angle must be formed in fp64 (an fp32 product is off by ~1e-2 rad)."""
    x = torch.randn(2, 300, 4, 64, generator=torch.Generator().manual_seed(pos0)).to(torch.bfloat16)
    y = atma.atma_rope(x.cuda(), 10000.0, pos0)
    torch.cuda.synchronize()
    e = out_err(to_np(y), oracle.rope(x, 10000.0, pos0), "bf16")  # beyond one bf16 rounding of the result
    note(f"  rope pos0={pos0} err={e:.3e}")
    assert e <= 1e-3


@pytest.mark.parametrize("B,T,Hq,Hkv,theta,D", [(1, 1, 1, 1, 0.0, 64), (2, 300, 4, 2, 0.0, 64),
                                                (1, 513, 3, 1, 10000.0, 64), (2, 2048, 16, 16, 10000.0, 64),
                                                (1, 777, 8, 2, 500.0, 64), (2, 1024, 8, 2, 10000.0, 128),
                                                (1, 300, 8, 2, 0.0, 128)])
def test_softmax_attn_fwd(atma, B, T, Hq, Hkv, theta, D):
    inp = workloads.make_polar_inputs(B, T, Hq, Hkv, D, seed=T + Hq)
    o = atma.atma_softmax_attn_fwd(inp["q"].cuda(), inp["k"].cuda(), inp["v"].cuda(), theta)
    torch.cuda.synchronize()
    go = to_np(o)
    assert np.all(np.isfinite(go))
    if theta == 0.0:
        e = rel_err_rows_bf16(go, oracle.softmax_attn(inp["q"], inp["k"], inp["v"]))
        note(f"  nope attn B{B} T{T} Hq{Hq} Hkv{Hkv} D{D} err={e:.3e}")
        assert e <= TOL["bf16"]
        return
    # exact rotation, with the operand-rounding tolerance allowed; on the first sequence and the
    # query heads of the first two kv heads when the case is large (the tolerance costs T^2 D^2)
    nb, nh = (1, 2 * (Hq // Hkv)) if B * Hq * T * D > 2 ** 20 else (B, Hq)
    hk = nh // (Hq // Hkv)
    ref, tol = oracle.softmax_attn(inp["q"][:nb, :, :nh], inp["k"][:nb, :, :hk], inp["v"][:nb, :, :hk],
                                   rope_theta=theta, tol_lambda=7.0)
    e_exact = rel_err_rows_bf16(go[:nb, :, :nh], ref, allow=tol)
    # the composition the library performs: bf16 rotation (atma_rope's output type), then NoPE
    rq = oracle.rope(inp["q"], theta, bf16=True)
    rk = oracle.rope(inp["k"], theta, bf16=True)
    e_comp = rel_err_rows_bf16(go, oracle.softmax_attn(rq, rk, inp["v"]))
    note(f"  rope attn B{B} T{T} Hq{Hq} Hkv{Hkv} theta={theta} D{D} err_exact={e_exact:.3e} err_comp={e_comp:.3e}")
    assert e_exact <= TOL["bf16"] and e_comp <= TOL["bf16"], (e_exact, e_comp)


@pytest.mark.parametrize("B,L,Lmax,Hq,Hkv,theta,D", [(1, 1, 1, 16, 16, 0.0, 64), (2, 1000, 1200, 16, 16, 10000.0, 64),
                                                     (3, 5000, 5000, 8, 2, 10000.0, 64), (4, 300, 512, 4, 4, 0.0, 64),
                                                     (2, 3000, 3000, 8, 2, 10000.0, 128)])
def test_softmax_attn_decode(atma, B, L, Lmax, Hq, Hkv, theta, D):
    """RoPE decode: the cache holds the keys rotated to their slots (oracle rope with bf16 output,
    the same values go to the GPU); the kernel rotates the query."""
    inp = workloads.make_decode_inputs(B, L, Hq=Hq, Hkv=Hkv, D=D, Lmax=Lmax, seed=L + Hq)
    kc = inp["k_cache"]
    if theta > 0:
        kc = torch.from_numpy(oracle.rope(kc, theta, bf16=True)).to(torch.bfloat16)
    o = atma.atma_softmax_attn_decode(inp["q"].cuda(), kc.cuda(), inp["v_cache"].cuda(), L, theta)
    torch.cuda.synchronize()
    ref = oracle.softmax_decode(inp["q"], kc, inp["v_cache"], L, rope_theta=theta)
    e = rel_err_rows_bf16(to_np(o), ref)
    note(f"  softmax decode B{B} L{L} Hq{Hq} Hkv{Hkv} theta={theta} err={e:.3e}")
    assert e <= TOL["bf16"]


def test_softmax_decode_is_last_prefill_row(atma):
    B, T, H = 2, 1500, 4
    inp = workloads.make_polar_inputs(B, T, H, H, 64, seed=8)
    q, k, v = (inp[x].cuda() for x in ("q", "k", "v"))
    o = atma.atma_softmax_attn_fwd(q, k, v, 10000.0)
    od = atma.atma_softmax_attn_decode(q[:, T - 1].contiguous(), atma.atma_rope(k, 10000.0), v, T, 10000.0)
    torch.cuda.synchronize()
    assert rel_err_rows_bf16(to_np(od), to_np(o[:, T - 1])) <= TOL["bf16"]
