"""GPU parity of the NoPE / RoPE control cores (causal softmax attention, rotary embedding)
against the fp64 oracle.  Budget: 2e-2 beyond one bf16 ulp, per output row against the row's
own RMS (plain softmax rows shrink ~1/sqrt(keys seen); see parity.rel_err_rows_bf16).  For
RoPE the rotated q and k are bf16 values on both sides (they are bf16 MFMA operands and a RoPE
KV cache stores them in bf16); rounding them alone moves the exact-rotation result by 2-6%."""
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
    # RoPE: the rotated q and k are bf16 operands (defined so; see the oracle)
    ref = oracle.softmax_attn(inp["q"], inp["k"], inp["v"], rope_theta=theta, rotated_bf16=True)
    e = rel_err_rows_bf16(to_np(o), ref)
    note(f"  softmax attn B{B} T{T} Hq{Hq} Hkv{Hkv} theta={theta} err={e:.3e}")
    assert e <= TOL["bf16"]


@pytest.mark.parametrize("B,L,Lmax,Hq,Hkv,theta,D", [(1, 1, 1, 16, 16, 0.0, 64), (2, 1000, 1200, 16, 16, 10000.0, 64),
                                                     (3, 5000, 5000, 8, 2, 10000.0, 64), (4, 300, 512, 4, 4, 0.0, 64),
                                                     (2, 3000, 3000, 8, 2, 10000.0, 128)])
def test_softmax_attn_decode(atma, B, L, Lmax, Hq, Hkv, theta, D):
    """RoPE decode: the library rotates the raw keys into the cache (atma_rope), the oracle
    rotates them itself."""
    inp = workloads.make_decode_inputs(B, L, Hq=Hq, Hkv=Hkv, D=D, Lmax=Lmax, seed=L + Hq)
    kc = inp["k_cache"].cuda()
    if theta > 0:
        kc = atma.atma_rope(kc, theta)
    o = atma.atma_softmax_attn_decode(inp["q"].cuda(), kc, inp["v_cache"].cuda(), L, theta)
    torch.cuda.synchronize()
    ref = oracle.softmax_decode(inp["q"], inp["k_cache"], inp["v_cache"], L, rope_theta=theta, rotated_keys_bf16=True)
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
