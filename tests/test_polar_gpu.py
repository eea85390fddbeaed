"""GPU parity of the Polar attention entry points against the fp64 oracle.

Prefill: every row at small sizes; at the long workloads a seeded sample of rows
(first and last rows, rows around every 256-query tile and 64-key block boundary,
random rows), which the oracle computes one by one (rows are independent).
Decode: the last causal row for a KV cache, against the oracle and against the
prefill kernel's last row.  Error = max |gpu - oracle| / rms(oracle) <= 2e-2 (bf16).
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


def _cpu_params(p):
    return {k: (v.cpu() if torch.is_tensor(v) else v) for k, v in p.items()}


def _dev_params(p):
    return {k: (v.cuda() if torch.is_tensor(v) else v) for k, v in p.items()}


def _check_prefill(atma, inp, rows=None, tag=""):
    q, k, v = (inp[x].cuda() for x in ("q", "k", "v"))
    o, mu, meff = atma.atma_polar_attn_fwd(q, k, v, _dev_params(inp["params"]), want_mu=True)
    torch.cuda.synchronize()
    for t in (o, mu, meff):  # every element written (the buffers start as NaN in GPU tests)
        assert torch.isfinite(t.float()).all()
    ref = oracle.polar_fwd(inp["q"], inp["k"], inp["v"], _cpu_params(inp["params"]), rows=rows)
    idx = slice(None) if rows is None else rows
    go = to_np(o)[:, idx]
    gmu = to_np(mu).transpose(0, 2, 1)[:, idx]      # [B,T,Hq] like the oracle
    gme = to_np(meff).transpose(0, 2, 1)[:, idx]
    eo, emu, eme = out_err(go, ref["o"], "bf16"), rel_err(gmu, ref["mu"]), rel_err_elem(gme, ref["meff"])
    note(f"  polar {tag} err_o={eo:.3e} err_mu={emu:.3e} err_meff={eme:.3e}")
    assert eo <= TOL["bf16"] and emu <= TOL["bf16"] and eme <= TOL["bf16"], (eo, emu, eme)
    # bounded channels on the GPU output: 0 <= mu <= 1 and ||o|| = mu (direction has unit norm)
    assert np.all(gmu >= 0) and np.all(gmu <= 1)
    np.testing.assert_allclose(np.linalg.norm(go, axis=-1), gmu, rtol=2e-2, atol=2e-3)
    return o, mu


@pytest.mark.parametrize("B,T,Hq,Hkv", [(1, 1, 1, 1), (1, 77, 2, 2), (2, 300, 4, 2), (1, 513, 3, 1),
                                        (1, 256, 2, 2), (2, 64, 8, 8)])
def test_polar_small_all_rows(atma, B, T, Hq, Hkv):
    inp = workloads.make_polar_inputs(B, T, Hq, Hkv, 64, seed=T + Hq)
    _check_prefill(atma, inp, tag=f"B{B} T{T} Hq{Hq} Hkv{Hkv}")


@pytest.mark.parametrize("B,T,Hq,Hkv", [(1, 1, 1, 1), (1, 77, 8, 2), (2, 300, 8, 2), (1, 513, 4, 4), (1, 1000, 2, 1)])
def test_polar_d128_all_rows(atma, B, T, Hq, Hkv):
    """Head width 128, including the real-model layout of 8 query and 2 kv heads."""
    inp = workloads.make_polar_inputs(B, T, Hq, Hkv, 128, seed=T + 128 + Hq)
    _check_prefill(atma, inp, tag=f"D128 B{B} T{T} Hq{Hq} Hkv{Hkv}")


def test_polar_d128_gqa_layer_b8_t2k(atma):
    """The 378M-class model's attention layout at training length: B=8, T=2048, 8 query heads,
    2 kv heads, D=128 (sampled rows)."""
    inp = workloads.make_polar_inputs(8, 2048, 8, 2, 128, seed=378)
    _check_prefill(atma, inp, rows=sample_rows(2048), tag="D128 gqa b8 t2k")


def test_polar_layer_b8_t2k(atma):
    """378M-class layer at 2K: B=8, T=2048, Hq=16, d=64 (sampled rows)."""
    inp = workloads.make_workload("layer_b8_t2k")["polar"]
    _check_prefill(atma, inp, rows=sample_rows(2048), tag="layer_b8_t2k")


def test_polar_layer_b8_t2k_output_only(atma):
    """The layer call without the optional mu / m_eff outputs (the form a layer step uses): the
    same o, bit for bit, as the call that also writes them, and every element written."""
    inp = workloads.make_workload("layer_b8_t2k")["polar"]
    q, k, v = (inp[x].cuda() for x in ("q", "k", "v"))
    p = _dev_params(inp["params"])
    o1, mu1, me1 = atma.atma_polar_attn_fwd(q, k, v, p)
    o2, _, _ = atma.atma_polar_attn_fwd(q, k, v, p, want_mu=True)
    torch.cuda.synchronize()
    assert mu1 is None and me1 is None
    assert torch.isfinite(o1.float()).all()
    assert torch.equal(o1, o2)


def test_polar_prefill_b2_t16k_needle(atma):
    w = workloads.WORKLOADS["prefill_b2_t16k_needle"]
    inp = workloads.make_polar_inputs(w.B, w.T, w.polar_Hq, w.polar_Hkv, w.polar_D, needle_frac=w.needle_frac,
                                      seed=w.seed)
    _check_prefill(atma, inp, rows=sample_rows(w.T, n_random=12), tag="b2_t16k_needle")


def test_polar_prefill_b1_t64k(atma):
    w = workloads.WORKLOADS["prefill_b1_t64k"]
    inp = workloads.make_polar_inputs(w.B, w.T, w.polar_Hq, w.polar_Hkv, w.polar_D, seed=w.seed)
    _check_prefill(atma, inp, rows=sample_rows(w.T, n_random=8), tag="b1_t64k")


def test_polar_prefill_b1_t256k(atma):
    """Evaluation-length prefill: B=1, T=262144, Hq=16 (sampled rows)."""
    w = workloads.WORKLOADS["prefill_b1_t256k"]
    inp = workloads.make_polar_inputs(w.B, w.T, w.polar_Hq, w.polar_Hkv, w.polar_D, seed=w.seed)
    _check_prefill(atma, inp, rows=sample_rows(w.T, n_random=8), tag="b1_t256k")


def test_polar_deterministic(atma):
    inp = workloads.make_polar_inputs(2, 700, 4, 4, 64, seed=9)
    q, k, v = (inp[x].cuda() for x in ("q", "k", "v"))
    p = _dev_params(inp["params"])
    o1, _, _ = atma.atma_polar_attn_fwd(q, k, v, p)
    o2, _, _ = atma.atma_polar_attn_fwd(q, k, v, p)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


@pytest.mark.parametrize("B,L,Lmax,Hq,Hkv", [(1, 1, 1, 16, 16), (2, 1000, 1200, 16, 16), (3, 5000, 5000, 8, 2),
                                             (1, 129, 4096, 4, 4), (16, 2048, 2048, 16, 16)])
def test_polar_decode(atma, B, L, Lmax, Hq, Hkv):
    inp = workloads.make_decode_inputs(B, L, Hq=Hq, Hkv=Hkv, Lmax=Lmax, seed=L)
    o, mu = atma.atma_polar_attn_decode(inp["q"].cuda(), inp["k_cache"].cuda(), inp["v_cache"].cuda(), L,
                                        _dev_params(inp["params"]), want_mu=True)
    torch.cuda.synchronize()
    ref = oracle.polar_decode(inp["q"], inp["k_cache"], inp["v_cache"], L, _cpu_params(inp["params"]))
    eo, emu = out_err(to_np(o), ref["o"], "bf16"), rel_err(to_np(mu), ref["mu"])
    note(f"  polar decode B{B} L{L} Hq{Hq} Hkv{Hkv} err_o={eo:.3e} err_mu={emu:.3e}")
    assert eo <= TOL["bf16"] and emu <= TOL["bf16"]


@pytest.mark.parametrize("lens,Hq,Hkv,D", [([1, 77, 300, 513, 128, 1000], 4, 2, 64), ([2048, 5, 129, 256], 2, 2, 64),
                                            ([64], 3, 1, 64), ([700, 3, 1500], 8, 2, 128)])
def test_polar_fwd_varlen(atma, lens, Hq, Hkv, D):
    """Packed prefill: each sequence (all rows, its own causal positions) against the oracle
    run on that sequence alone."""
    total = sum(lens)
    inp = workloads.make_polar_inputs(1, total, Hq, Hkv, D, seed=total)
    q, k, v = (inp[x][0].contiguous() for x in ("q", "k", "v"))
    cu = torch.tensor([0] + list(np.cumsum(lens)), dtype=torch.int32, device="cuda")
    o, mu, meff = atma.atma_polar_attn_fwd_varlen(q.cuda(), k.cuda(), v.cuda(), cu, max(lens),
                                                  _dev_params(inp["params"]), want_mu=True)
    torch.cuda.synchronize()
    for si, (s0, s1) in enumerate(zip(cu[:-1].tolist(), cu[1:].tolist())):
        ref = oracle.polar_fwd(q[None, s0:s1], k[None, s0:s1], v[None, s0:s1], _cpu_params(inp["params"]))
        eo = out_err(to_np(o[None, s0:s1]), ref["o"], "bf16")
        emu = rel_err(to_np(mu[:, s0:s1]).T[None], ref["mu"])
        eme = rel_err_elem(to_np(meff[:, s0:s1]).T[None], ref["meff"])
        note(f"  polar varlen seq{si} T{s1 - s0} err_o={eo:.3e} err_mu={emu:.3e} err_meff={eme:.3e}")
        assert eo <= TOL["bf16"] and emu <= TOL["bf16"] and eme <= TOL["bf16"], (si, eo, emu, eme)


def test_polar_fwd_varlen_matches_fixed_and_skips_bad_offsets(atma):
    """Equal lengths packed give exactly the fixed-length result; a sequence whose offsets are
    malformed is skipped (its rows keep their previous contents) and the others are unchanged."""
    B, T, H = 3, 700, 4
    inp = workloads.make_polar_inputs(B, T, H, H, 64, seed=33)
    q, k, v = (inp[x].cuda() for x in ("q", "k", "v"))
    p = _dev_params(inp["params"])
    of, muf, mef = atma.atma_polar_attn_fwd(q, k, v, p, want_mu=True)
    qp, kp, vp = (x.reshape(B * T, H, 64) for x in (q, k, v))
    cu = torch.tensor([0, T, 2 * T, 3 * T], dtype=torch.int32, device="cuda")
    op, mup, mep = atma.atma_polar_attn_fwd_varlen(qp, kp, vp, cu, T, p, want_mu=True)
    torch.cuda.synchronize()
    assert torch.equal(op.reshape(B, T, H, 64), of)
    assert torch.equal(mup.reshape(H, B, T).permute(1, 0, 2), muf)
    assert torch.equal(mep.reshape(H, B, T).permute(1, 0, 2), mef)
    # sequence 1 ends past the packed rows, sequence 2 runs backwards: both skipped, their rows
    # keep the sentinel; sequence 0 is computed as before
    for bad, bound in (([0, T, 5 * T, 3 * T], T), ([0, T, 3 * T], T)):  # second: length 2T > bound
        cb = torch.tensor(bad, dtype=torch.int32, device="cuda")
        ob, _, _ = atma.atma_polar_attn_fwd_varlen(qp, kp, vp, cb, bound, p, o=torch.full_like(qp, 7.0))
        torch.cuda.synchronize()
        assert torch.equal(ob[:T], op[:T])
        assert (ob[T:].float() == 7.0).all()


@pytest.mark.parametrize("B,L,Lmax,Hq,Hkv", [(1, 1, 1, 8, 2), (2, 1000, 1200, 8, 2), (3, 5000, 5000, 8, 2),
                                            (1, 20000, 20000, 16, 16), (4, 129, 4096, 4, 1)])
def test_polar_decode_d128(atma, B, L, Lmax, Hq, Hkv):
    inp = workloads.make_decode_inputs(B, L, Hq=Hq, Hkv=Hkv, D=128, Lmax=Lmax, seed=L + 128)
    o, mu = atma.atma_polar_attn_decode(inp["q"].cuda(), inp["k_cache"].cuda(), inp["v_cache"].cuda(), L,
                                        _dev_params(inp["params"]), want_mu=True)
    torch.cuda.synchronize()
    ref = oracle.polar_decode(inp["q"], inp["k_cache"], inp["v_cache"], L, _cpu_params(inp["params"]))
    eo, emu = out_err(to_np(o), ref["o"], "bf16"), rel_err(to_np(mu), ref["mu"])
    note(f"  polar decode D128 B{B} L{L} Hq{Hq} Hkv{Hkv} err_o={eo:.3e} err_mu={emu:.3e}")
    assert eo <= TOL["bf16"] and emu <= TOL["bf16"]


def test_polar_d128_decode_equals_prefill_last_row(atma):
    B, T, Hq, Hkv = 2, 1500, 8, 2
    inp = workloads.make_polar_inputs(B, T, Hq, Hkv, 128, seed=22)
    q, k, v = (inp[x].cuda() for x in ("q", "k", "v"))
    p = _dev_params(inp["params"])
    o, mu, _ = atma.atma_polar_attn_fwd(q, k, v, p, want_mu=True)
    od, mud = atma.atma_polar_attn_decode(q[:, T - 1].contiguous(), k, v, T, p, want_mu=True)
    torch.cuda.synchronize()
    assert out_err(to_np(od), to_np(o[:, T - 1]), "bf16") <= TOL["bf16"]
    assert rel_err(to_np(mud), to_np(mu[:, :, T - 1])) <= TOL["bf16"]


@pytest.mark.parametrize("lens,Lmax,Hq,Hkv", [([1, 77, 1000, 4096], 4096, 16, 16), ([300, 5, 2048], 2048, 8, 2),
                                               ([64, 63, 65, 129, 1, 200], 256, 4, 4)])
def test_polar_decode_varlen(atma, lens, Lmax, Hq, Hkv):
    """Heterogeneous batch: sequence b sees its own cache length; each row is checked against
    the oracle run on that sequence alone."""
    B = len(lens)
    inp = workloads.make_decode_inputs(B, Lmax, Hq=Hq, Hkv=Hkv, Lmax=Lmax, seed=B + Lmax)
    dl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    o, mu = atma.atma_polar_attn_decode_varlen(inp["q"].cuda(), inp["k_cache"].cuda(), inp["v_cache"].cuda(), dl,
                                               max(lens), _dev_params(inp["params"]), want_mu=True)
    torch.cuda.synchronize()
    for bi, L in enumerate(lens):
        ref = oracle.polar_decode(inp["q"][bi:bi + 1], inp["k_cache"][bi:bi + 1], inp["v_cache"][bi:bi + 1], L,
                                  _cpu_params(inp["params"]))
        eo, emu = out_err(to_np(o[bi:bi + 1]), ref["o"], "bf16"), rel_err(to_np(mu[bi:bi + 1]), ref["mu"])
        note(f"  polar decode varlen b{bi} L{L} err_o={eo:.3e} err_mu={emu:.3e}")
        assert eo <= TOL["bf16"] and emu <= TOL["bf16"], (bi, L, eo, emu)


def test_polar_decode_varlen_matches_uniform_and_flags_bad_lengths(atma):
    """Equal lengths give exactly the uniform-length result; a length outside [1, bound] turns
    only that sequence's outputs into NaN."""
    B, L, Lmax = 4, 3000, 4096
    inp = workloads.make_decode_inputs(B, Lmax, Lmax=Lmax, device="cuda", seed=5)
    p = _dev_params(inp["params"])
    ou, muu = atma.atma_polar_attn_decode(inp["q"], inp["k_cache"], inp["v_cache"], L, p, want_mu=True)
    dl = torch.full((B,), L, dtype=torch.int32, device="cuda")
    ov, muv = atma.atma_polar_attn_decode_varlen(inp["q"], inp["k_cache"], inp["v_cache"], dl, L, p, want_mu=True)
    torch.cuda.synchronize()
    assert torch.equal(ou, ov) and torch.equal(muu, muv)
    bad = torch.tensor([L, 0, L + 1, L], dtype=torch.int32, device="cuda")
    ob, mub = atma.atma_polar_attn_decode_varlen(inp["q"], inp["k_cache"], inp["v_cache"], bad, L, p, want_mu=True)
    torch.cuda.synchronize()
    assert torch.isnan(ob[1:3].float()).all() and torch.isnan(mub[1:3]).all()
    assert torch.equal(ob[[0, 3]], ou[[0, 3]]) and torch.equal(mub[[0, 3]], muu[[0, 3]])


def test_polar_decode_equals_prefill_last_row(atma):
    B, T, H = 2, 1500, 4
    inp = workloads.make_polar_inputs(B, T, H, H, 64, seed=21)
    q, k, v = (inp[x].cuda() for x in ("q", "k", "v"))
    p = _dev_params(inp["params"])
    o, mu, _ = atma.atma_polar_attn_fwd(q, k, v, p, want_mu=True)
    od, mud = atma.atma_polar_attn_decode(q[:, T - 1].contiguous(), k, v, T, p, want_mu=True)
    torch.cuda.synchronize()
    assert out_err(to_np(od), to_np(o[:, T - 1]), "bf16") <= TOL["bf16"]
    assert rel_err(to_np(mud), to_np(mu[:, :, T - 1])) <= TOL["bf16"]


def test_polar_decode_262k_context(atma):
    """Evaluation-length decode: one query against a 262144-token cache, B=1, Hq=Hkv=16."""
    L = workloads.DECODE_CONTEXT
    inp = workloads.make_decode_inputs(1, L, device="cuda", seed=0)
    o, mu = atma.atma_polar_attn_decode(inp["q"], inp["k_cache"], inp["v_cache"], L, inp["params"], want_mu=True)
    torch.cuda.synchronize()
    ref = oracle.polar_decode(inp["q"].cpu(), inp["k_cache"].cpu(), inp["v_cache"].cpu(), L,
                              _cpu_params(inp["params"]))
    eo, emu = out_err(to_np(o), ref["o"], "bf16"), rel_err(to_np(mu), ref["mu"])
    note(f"  polar decode 262k err_o={eo:.3e} err_mu={emu:.3e}")
    assert eo <= TOL["bf16"] and emu <= TOL["bf16"]


def test_polar_decode_262k_context_b16(atma):
    """Evaluation-length decode at batch 16 (262144-token caches); sequences 0 and 11 are checked
    against the oracle (sequences are independent)."""
    L = workloads.DECODE_CONTEXT
    inp = workloads.make_decode_inputs(16, L, device="cuda", seed=3)
    o, mu = atma.atma_polar_attn_decode(inp["q"], inp["k_cache"], inp["v_cache"], L, inp["params"], want_mu=True)
    torch.cuda.synchronize()
    idx = [0, 11]
    ref = oracle.polar_decode(inp["q"][idx].cpu(), inp["k_cache"][idx].cpu(), inp["v_cache"][idx].cpu(), L,
                              _cpu_params(inp["params"]))
    eo, emu = out_err(to_np(o[idx]), ref["o"], "bf16"), rel_err(to_np(mu[idx]), ref["mu"])
    note(f"  polar decode 262k b16 err_o={eo:.3e} err_mu={emu:.3e}")
    assert eo <= TOL["bf16"] and emu <= TOL["bf16"]
