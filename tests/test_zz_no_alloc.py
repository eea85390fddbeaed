"""The allocation-free Polar decode entry point (atma_polar_attn_decode_noalloc), called through
the C ABI, gives bitwise the result of atma_polar_attn_decode (same kernels, same split grid,
the split records in the library's fixed per-device array instead of a workspace), on two calls
in a row, the second with a smaller input; and it rejects a call that needs more than the array
holds, before launching.  Both results are also checked against the fp64 oracle."""
import ctypes

import pytest
import torch

import oracle
import workloads
from parity import TOL, note, out_err, rel_err, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def atma():
    import gated_delta_memory_amd as g

    assert torch.cuda.is_available()
    return g


def _call_noalloc(atma, inp, L, o, mu):
    """atma_polar_attn_decode_noalloc through ctypes, no Python-side allocation."""
    q, kc, vc = inp["q"], inp["k_cache"], inp["v_cache"]
    B, Hq, D = q.shape
    Lmax, Hkv = kc.shape[1], kc.shape[2]
    p = atma.polar_params_struct(inp["params"], Hq, D)
    st = atma.lib.atma_polar_attn_decode_noalloc(
        ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(kc.data_ptr()), ctypes.c_void_p(vc.data_ptr()), L, Lmax,
        ctypes.byref(p), ctypes.c_void_p(o.data_ptr()), ctypes.c_void_p(mu.data_ptr()), B, Hq, Hkv, D,
        atma.ATMA_BF16, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return st


@pytest.mark.parametrize("first,second", [((4, 20000, 16, 16, 64), (2, 3000, 16, 16, 64)),
                                          ((3, 9000, 8, 2, 128), (1, 129, 8, 2, 128))])
def test_noalloc_decode_equals_decode_twice(atma, first, second):
    for tag, (B, L, Hq, Hkv, D) in (("first", first), ("second", second)):
        inp = workloads.make_decode_inputs(B, L, Hq=Hq, Hkv=Hkv, D=D, seed=L + B)
        dev = {"q": inp["q"].cuda(), "k_cache": inp["k_cache"].cuda(), "v_cache": inp["v_cache"].cuda(),
               "params": {n: (x.cuda() if torch.is_tensor(x) else x) for n, x in inp["params"].items()}}
        o_ref, mu_ref = atma.atma_polar_attn_decode(dev["q"], dev["k_cache"], dev["v_cache"], L, dev["params"],
                                                    want_mu=True)
        o = torch.full((B, Hq, D), float("nan"), dtype=torch.bfloat16, device="cuda")
        mu = torch.full((B, Hq), float("nan"), device="cuda")
        assert _call_noalloc(atma, dev, L, o, mu) == atma.ATMA_OK
        torch.cuda.synchronize()
        ref = oracle.polar_decode(inp["q"], inp["k_cache"], inp["v_cache"], L, inp["params"])
        eo, emu = out_err(to_np(o), ref["o"], "bf16"), rel_err(to_np(mu), ref["mu"])
        note(f"  noalloc decode {tag} B{B} L{L} Hq{Hq} Hkv{Hkv} D{D}: err_o={eo:.3e} err_mu={emu:.3e}")
        assert torch.equal(o, o_ref) and torch.equal(mu, mu_ref)
        assert eo <= TOL["bf16"] and emu <= TOL["bf16"]


def test_noalloc_decode_rejects_oversize_before_launch(atma):
    """B = 512 sequences of 64 query heads at D = 128 need 512 * 64 * 132 * 4 B = 17.3 MB of split
    records, beyond the 16 MiB array: the call returns ATMA_ERR_WORKSPACE and leaves o untouched."""
    B, Hq, Hkv, D, L = 512, 64, 8, 128, 128
    assert atma.atma_polar_attn_decode_workspace_bytes(B, Hq, L, D) > 16 << 20
    q = torch.zeros(B, Hq, D, dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros(B, L, Hkv, D, dtype=torch.bfloat16, device="cuda")
    params = {n: (x.cuda() if torch.is_tensor(x) else x) for n, x in workloads.polar_params(Hq, D).items()}
    o = torch.full((B, Hq, D), 3.0, dtype=torch.bfloat16, device="cuda")
    mu = torch.full((B, Hq), 3.0, device="cuda")
    st = _call_noalloc(atma, {"q": q, "k_cache": kc, "v_cache": kc, "params": params}, L, o, mu)
    torch.cuda.synchronize()
    assert st == atma.ATMA_ERR_WORKSPACE
    assert (o.float() == 3.0).all() and (mu == 3.0).all()
