"""GPU parity of the gated-delta memory entry points against the fp64 oracle.

The HIP path is called through the C ABI (``gated_delta_memory_amd``) on seeded inputs;
the oracle runs the sequential recurrence (ATMA paper, Section 3.3 equation) on exact
copies of the same inputs.  Error = max |gpu - oracle| / rms(oracle); budgets 1e-4 (fp32)
and 2e-2 (bf16 inputs, fp32 state).
"""
import numpy as np
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


def _run_and_check(atma, inp, dtype, init=None, tag=""):
    q, k, v, a, b = (inp[x].cuda() for x in ("q", "k", "v", "alpha", "beta"))
    init_d = None if init is None else init.cuda()
    o, S = atma.atma_gdn_fwd(q, k, v, a, b, init_d)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(S).all()  # every element written
    ro, rS = oracle.gdn_sequential(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], init_state=init)
    eo, eS = out_err(to_np(o), ro, dtype), rel_err(to_np(S), rS)
    note(f"  gdn {tag} dtype={dtype} err_o={eo:.3e} err_S={eS:.3e}")
    assert eo <= TOL[dtype] and eS <= TOL[dtype], (eo, eS)
    return o, S


def test_gdn_f32_t256_d64(atma):
    """Memory only, fp32, B=1, H=1, T=256, d=64, chunk 64, seed 0."""
    inp = workloads.make_workload("gdn_t256_d64_f32")["gdn"]
    _run_and_check(atma, inp, "f32", tag="t256_d64")


@pytest.mark.parametrize("B,T,H,Dk,Dv,dtype", [
    (1, 1, 1, 64, 64, "f32"), (1, 63, 2, 64, 128, "f32"), (2, 200, 1, 128, 64, "f32"), (1, 129, 2, 128, 128, "f32"),
    (1, 1, 1, 128, 128, "bf16"), (2, 100, 3, 128, 128, "bf16"), (1, 64, 2, 64, 128, "bf16"),
    (1, 333, 2, 128, 64, "bf16"), (3, 65, 1, 64, 64, "bf16"),
])
def test_gdn_shapes_with_initial_state(atma, B, T, H, Dk, Dv, dtype):
    inp = workloads.make_gdn_inputs(B, T, H, Dk, Dv, dtype=dtype, seed=B * 1000 + T)
    init = torch.randn(B, H, Dv, Dk, generator=torch.Generator().manual_seed(T)) * 0.3
    _run_and_check(atma, inp, dtype, init=init, tag=f"B{B} T{T} H{H} Dk{Dk} Dv{Dv}")


@pytest.mark.parametrize("B,T,H,Dk,Dv", [(1, 2000, 2, 128, 128), (1, 1500, 1, 64, 128), (2, 1000, 1, 128, 64),
                                         (1, 4096, 1, 64, 64)])
def test_gdn_segmented_carry(atma, B, T, H, Dk, Dv):
    """Few (batch, head) pairs over many chunks: the library cuts the sequence into segments
    (summary pass, fp32 scan of the segment maps, parallel carry); every row is checked, with
    an initial state and a ragged last chunk where T is not a multiple of 64."""
    inp = workloads.make_gdn_inputs(B, T, H, Dk, Dv, dtype="bf16", seed=T + Dk)
    init = torch.randn(B, H, Dv, Dk, generator=torch.Generator().manual_seed(T + 1)) * 0.3
    _run_and_check(atma, inp, "bf16", init=init, tag=f"segmented B{B} T{T} H{H} Dk{Dk} Dv{Dv}")


def test_gdn_segmented_carry_long_memory(atma):
    """Segmented carry with gates close to 1 (alpha in (0.998, 1), small beta), so a segment's
    start state still weighs in thousands of tokens later and the fp32 scan of the segment
    maps (S_start A_seg + B_seg) is what the result depends on."""
    B, T, H, D = 1, 4096, 2, 128
    inp = workloads.make_gdn_inputs(B, T, H, D, dtype="bf16", seed=11)
    gen = torch.Generator().manual_seed(12)
    inp["alpha"] = 1.0 - 0.002 * torch.rand(B, T, H, generator=gen)
    inp["beta"] = torch.sigmoid(torch.randn(B, T, H, generator=gen) - 2.0)
    init = torch.randn(B, H, D, D, generator=gen) * 0.3
    _run_and_check(atma, inp, "bf16", init=init, tag="segmented long memory")


def test_gdn_layer_b8_t2k(atma):
    """378M-class layer at 2K: B=8, T=2048, H=8, d=128, bf16 inputs."""
    inp = workloads.make_workload("layer_b8_t2k")["gdn"]
    _run_and_check(atma, inp, "bf16", tag="layer_b8_t2k")


def test_gdn_prefill_b2_t16k_needle(atma):
    """B=2, T=16384, H=8, d=128 with 10% planted repeated needle keys."""
    w = workloads.WORKLOADS["prefill_b2_t16k_needle"]
    inp = workloads.make_gdn_inputs(w.B, w.T, w.gdn_H, w.gdn_D, dtype=w.dtype, needle_frac=w.needle_frac,
                                    seed=w.seed)
    _run_and_check(atma, inp, "bf16", tag="b2_t16k_needle")


def test_gdn_prefill_b1_t64k(atma):
    """B=1, T=65536, H=8, d=128: the full sequence against the sequential oracle."""
    w = workloads.WORKLOADS["prefill_b1_t64k"]
    inp = workloads.make_gdn_inputs(w.B, w.T, w.gdn_H, w.gdn_D, dtype=w.dtype, seed=w.seed)
    _run_and_check(atma, inp, "bf16", tag="b1_t64k")


def test_gdn_prefill_b1_t256k(atma):
    """Evaluation-length prefill: B=1, T=262144, H=8, d=128, all heads against the sequential oracle."""
    w = workloads.WORKLOADS["prefill_b1_t256k"]
    inp = workloads.make_gdn_inputs(w.B, w.T, w.gdn_H, w.gdn_D, dtype=w.dtype, seed=w.seed)
    _run_and_check(atma, inp, "bf16", tag="b1_t256k")


def test_gdn_resume_equals_one_pass(atma):
    """prefill(T1) then prefill(T2, init=final) equals prefill(T1+T2) (state carry across calls)."""
    inp = workloads.make_gdn_inputs(2, 300, 2, 128, 128, dtype="bf16", seed=7)
    d = {x: t.cuda() for x, t in inp.items()}
    o, S = atma.atma_gdn_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"])
    T1 = 130
    part = lambda s: [d[x][:, s].contiguous() for x in ("q", "k", "v", "alpha", "beta")]
    o1, S1 = atma.atma_gdn_fwd(*part(slice(0, T1)))
    o2, S2 = atma.atma_gdn_fwd(*part(slice(T1, None)), S1)
    torch.cuda.synchronize()
    ro, rS = oracle.gdn_sequential(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"])
    e1 = out_err(to_np(torch.cat([o1, o2], dim=1)), ro, "bf16")
    e2 = rel_err(to_np(S2), rS)
    note(f"  gdn resume err_o={e1:.3e} err_S={e2:.3e}")
    assert e1 <= TOL["bf16"] and e2 <= TOL["bf16"]


def test_gdn_final_state_may_alias_init(atma):
    inp = workloads.make_gdn_inputs(1, 90, 2, 64, 64, dtype="f32", seed=3)
    d = {x: t.cuda() for x, t in inp.items()}
    init = torch.randn(1, 2, 64, 64, generator=torch.Generator().manual_seed(1))
    S = init.clone().cuda()
    o, S_out = atma.atma_gdn_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], S, final_state=S)
    torch.cuda.synchronize()
    assert S_out.data_ptr() == S.data_ptr()
    ro, rS = oracle.gdn_sequential(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], init_state=init)
    assert rel_err(to_np(S), rS) <= TOL["f32"]
    assert rel_err(to_np(o), ro) <= TOL["f32"]


def test_gdn_deterministic(atma):
    """No atomics: two runs agree bit for bit."""
    inp = workloads.make_gdn_inputs(2, 257, 4, 128, 128, dtype="bf16", seed=11)
    d = [t.cuda() for t in (inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"])]
    o1, S1 = atma.atma_gdn_fwd(*d)
    o2, S2 = atma.atma_gdn_fwd(*d)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


@pytest.mark.parametrize("B,H,Dk,Dv,dtype", [(1, 8, 128, 128, "bf16"), (16, 8, 128, 128, "bf16"),
                                            (2, 3, 64, 128, "f32"), (1, 1, 128, 64, "f32")])
def test_gdn_decode_step(atma, B, H, Dk, Dv, dtype):
    """One step against the oracle, then a run of steps against the prefill of the same tokens."""
    gen = torch.Generator().manual_seed(B * 100 + H)
    td = workloads.torch_dtype(dtype)
    unit = lambda x: x / x.norm(dim=-1, keepdim=True)
    q = unit(torch.randn(B, H, Dk, generator=gen)).to(td)
    k = unit(torch.randn(B, H, Dk, generator=gen)).to(td)
    v = torch.randn(B, H, Dv, generator=gen).to(td)
    a = torch.sigmoid(torch.randn(B, H, generator=gen) * 0.5 + 3)
    b = torch.sigmoid(torch.randn(B, H, generator=gen))
    S0 = torch.randn(B, H, Dv, Dk, generator=gen) * 0.1
    S = S0.clone().cuda()
    o = atma.atma_gdn_decode_step(q.cuda(), k.cuda(), v.cuda(), a.cuda(), b.cuda(), S)
    torch.cuda.synchronize()
    ro, rS = oracle.gdn_decode_step(q, k, v, a, b, S0)
    eo, eS = out_err(to_np(o), ro, dtype), rel_err(to_np(S), rS)
    note(f"  gdn decode B{B} H{H} {dtype} err_o={eo:.3e} err_S={eS:.3e}")
    assert eo <= TOL[dtype] and eS <= TOL[dtype]


def test_gdn_decode_steps_match_prefill(atma):
    inp = workloads.make_gdn_inputs(2, 70, 2, 128, 128, dtype="f32", seed=5)
    d = {x: t.cuda() for x, t in inp.items()}
    o, S = atma.atma_gdn_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"])
    St = torch.zeros(2, 2, 128, 128, device="cuda")
    outs = []
    for t in range(70):
        outs.append(atma.atma_gdn_decode_step(*(d[x][:, t].contiguous() for x in ("q", "k", "v", "alpha", "beta")),
                                              St))
    torch.cuda.synchronize()
    assert rel_err(to_np(torch.stack(outs, dim=1)), to_np(o)) <= 1e-4
    assert rel_err(to_np(St), to_np(S)) <= 1e-4


def _packed(inp):
    """[1, total, ...] workload tensors as packed [total, ...] tensors on the GPU."""
    return [inp[x][0].contiguous().cuda() for x in ("q", "k", "v", "alpha", "beta")]


@pytest.mark.parametrize("lens,H,Dk,Dv", [([1, 64, 65, 300, 129], 2, 128, 128), ([4096, 100, 1500], 1, 64, 128),
                                          ([2000, 3], 2, 128, 64)])
def test_gdn_fwd_varlen(atma, lens, H, Dk, Dv):
    """Packed prefill: every sequence, from its own initial state, against the oracle's
    sequential recurrence on that sequence alone.  The long-and-short mixes make the library
    cut the carry into segments, most of them empty for the short sequences."""
    total = sum(lens)
    inp = workloads.make_gdn_inputs(1, total, H, Dk, Dv, dtype="bf16", seed=total + Dk)
    init = torch.randn(len(lens), H, Dv, Dk, generator=torch.Generator().manual_seed(total)) * 0.3
    q, k, v, a, b = _packed(inp)
    cu = torch.tensor([0] + list(np.cumsum(lens)), dtype=torch.int32, device="cuda")
    o, S = atma.atma_gdn_fwd_varlen(q, k, v, a, b, cu, max(lens), init.cuda())
    torch.cuda.synchronize()
    for si, (s0, s1) in enumerate(zip(cu[:-1].tolist(), cu[1:].tolist())):
        ro, rS = oracle.gdn_sequential(*(inp[x][:, s0:s1] for x in ("q", "k", "v", "alpha", "beta")),
                                       init_state=init[si:si + 1])
        eo, eS = out_err(to_np(o[None, s0:s1]), ro, "bf16"), rel_err(to_np(S[si:si + 1]), rS)
        note(f"  gdn varlen seq{si} T{s1 - s0} err_o={eo:.3e} err_S={eS:.3e}")
        assert eo <= TOL["bf16"] and eS <= TOL["bf16"], (si, eo, eS)


def test_gdn_fwd_varlen_matches_fixed_and_skips_bad_offsets(atma):
    """Equal lengths packed give exactly the fixed-length result; a sequence whose offsets are
    malformed is skipped (its rows and final state keep their previous contents)."""
    B, T, H, D = 2, 700, 2, 128
    inp = workloads.make_gdn_inputs(B, T, H, D, dtype="bf16", seed=44)
    q, k, v, a, b = (inp[x].cuda() for x in ("q", "k", "v", "alpha", "beta"))
    of, Sf = atma.atma_gdn_fwd(q, k, v, a, b)
    pk = [x.reshape(B * T, *x.shape[2:]) for x in (q, k, v, a, b)]
    cu = torch.tensor([0, T, 2 * T], dtype=torch.int32, device="cuda")
    op, Sp = atma.atma_gdn_fwd_varlen(*pk, cu, T)
    torch.cuda.synchronize()
    assert torch.equal(op.reshape(B, T, H, D), of) and torch.equal(Sp, Sf)
    for bad, bound in (([0, T, 5 * T], T), ([0, T, T - 1], T), ([0, T, 2 * T], T - 1)):
        cb = torch.tensor(bad, dtype=torch.int32, device="cuda")
        fin = torch.full_like(Sp, 7.0)
        ob, Sb = atma.atma_gdn_fwd_varlen(*pk, cb, max(bound, 1), o=torch.full_like(op, 7.0), final_state=fin)
        torch.cuda.synchronize()
        if bound == T:   # sequence 0 valid, sequence 1 malformed
            assert torch.equal(ob[:T], op[:T]) and torch.equal(Sb[0], Sp[0])
            assert (ob[T:].float() == 7.0).all() and (Sb[1] == 7.0).all()
        else:            # both sequences longer than the declared bound: nothing written
            assert (ob.float() == 7.0).all() and (Sb == 7.0).all()
