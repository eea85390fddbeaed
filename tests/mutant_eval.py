"""Evaluates the oracle build named by ATMA_ORACLE_LIB on the inputs of the GPU parity tests.

Used by test_metric_strength.py: that test builds copies of oracle.c with one planted mistake
each, runs this script against each copy in a subprocess, and scores the copy's results with the
GPU tests' own metrics against the correct oracle.  Usage:

    ATMA_ORACLE_LIB=... python tests/mutant_eval.py KIND OUT.npz

KIND names a group of cases (see CASES); every array of every case is written to OUT.npz under
"<case index>/<name>".  Not a test module (no test_ prefix); CPU only.
"""
import os
import sys

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.join(ROOT, "tests"))

import oracle  # noqa: E402
import workloads  # noqa: E402
from parity import sample_rows  # noqa: E402

# The cases of the GPU tests, with the same seeds (see the test named beside each group).
CASES = {
    # test_polar_bwd_gpu.test_polar_bwd_matches_oracle / _tile_edges (seed = 1000 + T + Hq + D / 4000 + T)
    "polar_bwd": [(1, 77, 2, 2, 64, 1143), (2, 300, 4, 2, 64, 1368), (1, 513, 3, 1, 64, 1580),
                  (1, 1024, 8, 2, 128, 2160), (1, 2048, 4, 2, 64, 3116), (1, 129, 2, 1, 64, 4129)],
    # test_gdn_bwd_gpu.test_gdn_bwd_matches_oracle (seed = 100 + T + Dk + Dv) and the 2K layer's batch 0
    "gdn_bwd": [(1, 77, 2, 64, 64, "bf16", True, True, 305), (2, 200, 2, 128, 128, "bf16", False, False, 556),
                (1, 130, 3, 64, 128, "f32", True, False, 422), (1, 1000, 1, 128, 128, "bf16", True, True, 1356),
                ("layer", 2048)],
    # test_polar_gpu: small all-row cases and the 2K layer's sampled rows
    "polar_fwd": [(2, 300, 4, 2, 64, 304), (1, 513, 3, 1, 64, 516), ("layer", 2048)],
    # test_gdn_gpu: the fp32 T=256 workload and the 2K layer (bf16)
    "gdn_fwd": [("gdn_t256_d64_f32",), ("layer_b8_t2k",)],
    # test_baseline_gpu.test_softmax_attn_fwd (seed = T + Hq) and test_softmax_attn_decode (seed = L + Hq)
    "softmax": [(2, 300, 4, 2, 0.0, 64, 304), (1, 513, 3, 1, 10000.0, 64, 516), (1, 777, 8, 2, 500.0, 64, 785),
                ("decode", 2, 1000, 1200, 16, 16, 10000.0, 64, 1016), ("decode", 4, 300, 512, 4, 4, 0.0, 64, 304)],
    # test_canon_gpu.test_canon_matches_oracle (seed = T + C + K)
    "canon": [(2, 300, 1024, 4, 1, 8, True), (3, 77, 256, 3, 0, 4, False), (2, 5, 512, 8, 1, 16, True)],
}


def polar_bwd_inputs(B, T, Hq, Hkv, D, seed):
    inp = workloads.make_polar_inputs(B, T, Hq, Hkv, D, seed=seed)
    do = torch.randn(B, T, Hq, D, generator=torch.Generator().manual_seed(seed + 1)).to(torch.bfloat16)
    return inp, do


def gdn_bwd_inputs(case):
    if case[0] == "layer":
        inp = workloads.make_workload("layer_b8_t2k")["gdn"]
        B, T, H, D = inp["q"].shape
        do = torch.randn(B, T, H, D, generator=torch.Generator().manual_seed(2049)).to(torch.bfloat16)
        one = {x: inp[x][:1] for x in ("q", "k", "v", "alpha", "beta")}
        return one, do[:1], None, None, "bf16"
    B, T, H, Dk, Dv, dtype, init, final, seed = case
    inp = workloads.make_gdn_inputs(B, T, H, Dk, Dv, dtype=dtype, seed=seed)
    gen = torch.Generator().manual_seed(seed + 7)
    do = torch.randn(B, T, H, Dv, generator=gen).to(workloads.torch_dtype(dtype))
    S0 = torch.randn(B, H, Dv, Dk, generator=gen) * 0.3 if init else None
    dSf = torch.randn(B, H, Dv, Dk, generator=gen) * 0.5 if final else None
    return inp, do, S0, dSf, dtype


def canon_inputs(B, T, C, K, res, heads, st):
    gen = torch.Generator().manual_seed(T + C + K)
    x = torch.randn(B, T, C, generator=gen).to(torch.bfloat16)
    w = torch.randn(K, C, generator=gen) * 0.5
    state = torch.randn(B, K - 1, C, generator=gen).to(torch.bfloat16) if st and K > 1 else None
    return x, w, state


def evaluate(kind):
    """{case index: {name: array}} of the oracle's results on the group's cases."""
    out = {}
    for i, c in enumerate(CASES[kind]):
        if kind == "polar_bwd":
            inp, do = polar_bwd_inputs(*c)
            out[i] = oracle.polar_bwd(inp["q"], inp["k"], inp["v"], inp["params"], do)
        elif kind == "gdn_bwd":
            inp, do, S0, dSf, _ = gdn_bwd_inputs(c)
            out[i] = oracle.gdn_bwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], do, init_state=S0,
                                    dS_final=dSf)
        elif kind == "polar_fwd":
            if c[0] == "layer":
                inp = workloads.make_workload("layer_b8_t2k")["polar"]
                rows = sample_rows(c[1])
            else:
                inp, rows = workloads.make_polar_inputs(*c[:5], seed=c[5]), None
            r = oracle.polar_fwd(inp["q"], inp["k"], inp["v"], inp["params"], rows=rows)
            out[i] = {"o": r["o"], "mu": r["mu"], "meff": r["meff"]}
        elif kind == "gdn_fwd":
            g = workloads.make_workload(c[0])["gdn"]
            o, S = oracle.gdn_sequential(g["q"], g["k"], g["v"], g["alpha"], g["beta"])
            out[i] = {"o": o, "S": S}
        elif kind == "softmax":
            if c[0] == "decode":
                _, B, L, Lmax, Hq, Hkv, theta, D, seed = c
                inp = workloads.make_decode_inputs(B, L, Hq=Hq, Hkv=Hkv, D=D, Lmax=Lmax, seed=seed)
                kc = inp["k_cache"]
                if theta > 0:
                    kc = oracle.rope(kc, theta, bf16=True)
                out[i] = {"o": oracle.softmax_decode(inp["q"], kc, inp["v_cache"], L, rope_theta=theta)}
            else:
                B, T, Hq, Hkv, theta, D, seed = c
                inp = workloads.make_polar_inputs(B, T, Hq, Hkv, D, seed=seed)
                res = {"o": oracle.softmax_attn(inp["q"], inp["k"], inp["v"], rope_theta=theta)}
                if theta > 0:
                    rq, rk = oracle.rope(inp["q"], theta, bf16=True), oracle.rope(inp["k"], theta, bf16=True)
                    res["o_comp"] = oracle.softmax_attn(rq, rk, inp["v"])
                out[i] = res
        elif kind == "canon":
            x, w, state = canon_inputs(*c)
            out[i] = {"y": oracle.canon(x, w, state=state, residual=bool(c[4]), heads=c[5])}
    return out


if __name__ == "__main__":
    kind, path = sys.argv[1], sys.argv[2]
    res = evaluate(kind)
    np.savez(path, **{f"{i}/{n}": np.asarray(a) for i, r in res.items() for n, a in r.items()})
