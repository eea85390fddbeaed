"""GPU parity at the method's degenerate and extreme cases, against the fp64 oracle.

Polar attention (Section 3.2 equation, Appendix A.2 channels, Appendix C.2 single softmax):
  * all values and the null value zero: s = 0, so the direction clamp max(||s||, eps) gives o = 0
    exactly while mu still follows the weights;
  * sharply peaked logits (q scaled by 4, exactly in bf16): the running origin moves many times;
  * a saturated magnitude (mag_beta = 5, mu -> 1);
  * the null switched off (null_bias = -1e4: one softmax over real keys only) and dominant
    (null_bias = +5: almost all mass on the null, small mu, direction near v_null);
  * head width 128 with more than 4096 query tiles, where the prefill runs one tile per workgroup
    instead of pairing the heaviest and lightest tiles.
Gated-delta memory (Section 3.3 equation):
  * beta = 0: pure decay, S_T = (prod alpha) S_0 and o_t = (prod_{s<=t} alpha_s) S_0 q_t;
  * alpha = beta = 1 with orthonormal keys (signed standard basis vectors, exact in bf16):
    querying a stored key returns its value exactly, also after a key is overwritten;
  * values and initial state scaled by 2^12 (entries up to ~2^14.2, near the 2^15 limit of the
    bf16 path's fp16 staging): the relative error must not change.
Budgets as everywhere: max |gpu - oracle| / rms(oracle) <= 2e-2 beyond the output cast (bf16) or
<= 1e-4 (fp32); m_eff per element.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import TOL, note, out_err, rel_err, rel_err_elem, sample_rows, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def atma():
    import gated_delta_memory_amd as g

    assert torch.cuda.is_available()
    return g


def _polar(atma, inp, rows=None, tag=""):
    q, k, v = (inp[x].cuda() for x in ("q", "k", "v"))
    pd = {n: (x.cuda() if torch.is_tensor(x) else x) for n, x in inp["params"].items()}
    o, mu, meff = atma.atma_polar_attn_fwd(q, k, v, pd, want_mu=True)
    torch.cuda.synchronize()
    for t in (o, mu, meff):
        assert torch.isfinite(t.float()).all(), "an output element was not written (NaN poison left)"
    ref = oracle.polar_fwd(inp["q"], inp["k"], inp["v"], inp["params"], rows=rows)
    idx = slice(None) if rows is None else rows
    go = to_np(o)[:, idx]
    gmu = to_np(mu).transpose(0, 2, 1)[:, idx]
    gme = to_np(meff).transpose(0, 2, 1)[:, idx]
    eo, emu, eme = out_err(go, ref["o"], "bf16"), rel_err(gmu, ref["mu"]), rel_err_elem(gme, ref["meff"])
    note(f"  polar edge {tag}: err_o={eo:.3e} err_mu={emu:.3e} err_meff={eme:.3e}")
    assert eo <= TOL["bf16"] and emu <= TOL["bf16"] and eme <= TOL["bf16"], (eo, emu, eme)
    return go, gmu, ref


def test_polar_zero_values_give_zero_output(atma):
    inp = workloads.make_polar_inputs(2, 300, 4, 2, 64, seed=501)
    inp["v"].zero_()
    inp["params"]["v_null"].zero_()
    go, gmu, ref = _polar(atma, inp, tag="v = v_null = 0")
    assert np.all(ref["o"] == 0.0) and np.all(go == 0.0)
    assert np.all(gmu >= 0)  # null-dominated rows may round mu to 0, as the oracle does


@pytest.mark.parametrize("D", [64, 128])
def test_polar_peaked_logits(atma, D):
    inp = workloads.make_polar_inputs(1, 1000, 4, 2, D, seed=502 + D)
    inp["q"] = (inp["q"].float() * 4).to(torch.bfloat16)  # exact: a power of two
    _polar(atma, inp, tag=f"q x 4, D={D}")


def test_polar_saturated_magnitude(atma):
    inp = workloads.make_polar_inputs(1, 700, 4, 4, 64, seed=503)
    inp["params"]["mag_beta"].fill_(5.0)
    go, gmu, ref = _polar(atma, inp, tag="mag_beta = 5")
    assert np.all(gmu <= 1.0) and np.mean(ref["mu"] > 0.99) > 0.45  # the real-dominated heads saturate


@pytest.mark.parametrize("bias", [-1e4, 5.0])
def test_polar_null_off_and_dominant(atma, bias):
    inp = workloads.make_polar_inputs(2, 513, 4, 2, 64, seed=504)
    inp["params"]["null_bias"].fill_(bias)
    go, gmu, ref = _polar(atma, inp, tag=f"null_bias = {bias}")
    if bias > 0:  # most of the mass on the null: the direction leans to v_null
        assert np.median(ref["meff"]) < 2.0


def test_polar_d128_unpaired_tiles(atma):
    """B=3, T=16384, 16 query / 2 kv heads at D=128: 3 * 128 * 16 = 6144 query tiles (> 4096), so
    every workgroup runs one tile (heaviest first); sampled rows."""
    inp = workloads.make_polar_inputs(3, 16384, 16, 2, 128, seed=505)
    _polar(atma, inp, rows=sample_rows(16384, n_random=6), tag="D128 6144 tiles")


# ---- gated-delta memory -------------------------------------------------------------------------
def _gdn(atma, inp, dtype, init, tag):
    q, k, v, a, b = (inp[x].cuda() for x in ("q", "k", "v", "alpha", "beta"))
    o, S = atma.atma_gdn_fwd(q, k, v, a, b, None if init is None else init.cuda())
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(S).all()
    ro, rS = oracle.gdn_sequential(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], init_state=init)
    eo, eS = out_err(to_np(o), ro, dtype), rel_err(to_np(S), rS)
    note(f"  gdn edge {tag} {dtype}: err_o={eo:.3e} err_S={eS:.3e}")
    assert eo <= TOL[dtype] and eS <= TOL[dtype], (eo, eS)
    return to_np(o), to_np(S), ro, rS


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_gdn_pure_decay(atma, dtype):
    inp = workloads.make_gdn_inputs(2, 300, 2, 128, 128, dtype=dtype, seed=506)
    inp["beta"].zero_()
    init = torch.randn(2, 2, 128, 128, generator=torch.Generator().manual_seed(507))
    go, gS, ro, rS = _gdn(atma, inp, dtype, init, "beta = 0")
    decay = np.prod(inp["alpha"].double().numpy(), axis=1)  # [B, H]
    assert np.allclose(rS, decay[:, :, None, None] * init.double().numpy(), rtol=1e-12, atol=0)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_gdn_exact_recall_orthonormal_keys(atma, dtype):
    """alpha = beta = 1, keys = signed standard basis vectors (each used twice, the second time with
    a new value), queries = the token's own key: o_t = v_t for every t."""
    B, H, D = 1, 2, 128
    T = 2 * D
    gen = torch.Generator().manual_seed(508)
    perm = torch.cat([torch.randperm(D, generator=gen), torch.randperm(D, generator=gen)])
    sign = torch.where(torch.rand(T, generator=gen) < 0.5, -1.0, 1.0)
    k = torch.zeros(B, T, H, D)
    k[0, torch.arange(T), :, perm] = sign[:, None]
    v = torch.randn(B, T, H, D, generator=gen)
    td = workloads.torch_dtype(dtype)
    inp = {"q": k.to(td), "k": k.to(td), "v": v.to(td), "alpha": torch.ones(B, T, H), "beta": torch.ones(B, T, H)}
    go, gS, ro, rS = _gdn(atma, inp, dtype, None, "alpha = beta = 1, orthonormal keys")
    assert np.allclose(ro, inp["v"].double().numpy(), rtol=0, atol=1e-12)


def test_gdn_values_near_fp16_staging_limit(atma):
    """Values and the initial state scaled by 2^12 (the bf16 path stages fp16 operands, which hold
    magnitudes below 2^15): the scaled result is the scaled result, within the same budget."""
    inp = workloads.make_gdn_inputs(2, 700, 2, 128, 128, dtype="bf16", seed=509)
    inp["v"] = (inp["v"].float() * 4096).to(torch.bfloat16)
    init = torch.randn(2, 2, 128, 128, generator=torch.Generator().manual_seed(510)) * 4096
    assert float(inp["v"].float().abs().max()) > 2 ** 14
    _gdn(atma, inp, "bf16", init, "v x 2^12")


def test_binding_buffers_are_guarded(atma):
    """The GPU tests' fixture hands the binding guarded, poisoned buffers (checked after each test)."""
    inp = workloads.make_gdn_inputs(1, 70, 1, 64, 64, seed=9)
    o, fs = atma.atma_gdn_fwd(*[inp[x].cuda() for x in ("q", "k", "v", "alpha", "beta")])
    torch.cuda.synchronize()
    assert len(atma.torch.guarded) >= 3  # o, the final state and the workspace
    assert torch.isfinite(o.float()).all() and torch.isfinite(fs).all()
