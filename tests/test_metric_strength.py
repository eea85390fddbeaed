"""The GPU parity metrics reject plausible mistakes (CPU only).

Every planted mistake of the oracle mutation suite that changes a result the GPU tests compare
against is built into a copy of oracle.c; the copy's results on the GPU tests' own inputs (same
shapes, seeds and sampled rows, T = 2048 included) stand for a GPU path that made that mistake,
and the GPU tests' own metrics and budgets (from parity.py) must reject them: a mistaken kernel
could not pass the GPU suite.  Kernel-independent rounding is not involved: the comparison is of
two fp64 results, so each score shows how far the mistake lies outside the budget.

Mistakes in oracle-only cross-checks (the chunked memory form, the streaming Polar form, the
rounding tolerance) are not GPU references and are covered by test_oracle_mutations.py alone.
"""
import os
import subprocess
import sys

import numpy as np
import pytest

from mutant_eval import CASES, evaluate
from parity import (POLAR_GRADS, TOL, gdn_grad_errors, gdn_grad_failures, out_err, polar_grad_errors,
                    polar_grad_failures, rel_err, rel_err_elem, rel_err_rows_bf16)
from test_oracle_mutations import MUTANTS, ROOT, SRC

KIND = {"gdn_bwd_": "gdn_bwd", "polar_bwd_": "polar_bwd", "gdn_": "gdn_fwd", "polar_": "polar_fwd",
        "rope_": "softmax", "softmax_": "softmax", "canon_": "canon"}
NOT_GPU_REFERENCES = {"gdn_chunk_decay_sign", "streaming_q2_rho_linear"}


def kind_of(name):
    for prefix, kind in KIND.items():  # longest prefixes first (dict order)
        if name.startswith(prefix):
            return kind
    return None


STRENGTH_MUTANTS = sorted(n for n in MUTANTS if kind_of(n) and n not in NOT_GPU_REFERENCES)
_REF = {}


def reference(kind):
    if kind not in _REF:
        _REF[kind] = evaluate(kind)
    return _REF[kind]


def case_rejects(kind, c, got, ref):
    """(rejected?, score text) of one case with the GPU test's metric for it."""
    if kind == "polar_bwd":
        errs = polar_grad_errors({n: got[n] for n in POLAR_GRADS}, ref)
        bad = polar_grad_failures(errs)
        return bool(bad), " ".join(f"{n}={e[0]:.1e}/{e[1]:.1e}" for n, e in bad.items())
    if kind == "gdn_bwd":
        dtype = "bf16" if c[0] == "layer" else c[5]
        names = ("dq", "dk", "dv", "dalpha", "dbeta") + (() if c[0] == "layer" else ("dinit",))
        bad = gdn_grad_failures(gdn_grad_errors(got, ref, names), dtype)
        return bool(bad), " ".join(f"{n}={e[0]:.1e}/{e[1]:.1e}" for n, e in bad.items())
    if kind == "polar_fwd":
        eo, emu, eme = out_err(got["o"], ref["o"], "bf16"), rel_err(got["mu"], ref["mu"]), rel_err_elem(
            got["meff"], ref["meff"])
        return max(eo, emu, eme) > TOL["bf16"], f"o={eo:.2e} mu={emu:.2e} meff={eme:.2e}"
    if kind == "gdn_fwd":
        dt = "f32" if "f32" in c[0] else "bf16"
        eo, eS = out_err(got["o"], ref["o"], dt), rel_err(got["S"], ref["S"])
        return max(eo, eS) > TOL[dt], f"o={eo:.2e} S={eS:.2e}"
    if kind == "softmax":
        e = rel_err_rows_bf16(got["o"], ref["o"])
        txt = f"o={e:.2e}"
        if "o_comp" in ref:
            ec = rel_err_rows_bf16(got["o_comp"], ref["o_comp"])
            txt += f" comp={ec:.2e}"
            e = max(e, ec)
        return e > TOL["bf16"], txt
    if kind == "canon":
        e = out_err(got["y"], ref["y"], "bf16")
        return e > TOL["bf16"], f"y={e:.2e}"
    raise ValueError(kind)


# A planted mistake can be invisible on a case by construction (the case never reaches the
# mutated term); those (mutant, case index) pairs are listed with the reason.
EXEMPT = {
    # RoPE mistakes cannot show on NoPE cases (theta = 0)
    **{(m, i): "NoPE case" for m in ("rope_reflect", "rope_half_frequency") for i in (0, 4)},
    # the decode query's position only matters with RoPE
    **{("softmax_decode_query_position", i): "not a RoPE decode case" for i in (0, 1, 2, 4)},
    # prefill mistakes cannot show on decode cases and vice versa
    **{(m, i): "decode case" for m in ("softmax_sees_next_key",) for i in (3, 4)},
    # a state mistake needs a carried state (these cases have none)
    **{("canon_state_offset", i): "no carried state" for i in (1,)},
}


def _run_mutant(name, workdir):
    """Builds the mutant and evaluates it on its group's cases; returns the npz path, or None when
    the mutant oracle refuses to run (then every case is caught)."""
    kind = kind_of(name)
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    d = workdir / name
    d.mkdir()
    (d / "m.c").write_text(src.replace(old, new))
    lib = d / "libm.so"
    subprocess.run(["gcc", "-O2", "-std=c99", "-fPIC", "-D_POSIX_C_SOURCE=200809L", "-shared", "-o", str(lib),
                    str(d / "m.c"), "-lm", "-lpthread"], check=True)
    out = d / "res.npz"
    r = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "mutant_eval.py"), kind, str(out)],
                       env=dict(os.environ, ATMA_ORACLE_LIB=str(lib)), cwd=ROOT, capture_output=True, text=True,
                       timeout=1800)
    return str(out) if r.returncode == 0 else None


@pytest.fixture(scope="module")
def mutant_results(tmp_path_factory):
    """Every mutant built and evaluated up front, one process per CPU (at most 8)."""
    import concurrent.futures as cf

    work = tmp_path_factory.mktemp("strength")
    with cf.ThreadPoolExecutor(max_workers=max(1, min(8, os.cpu_count() or 1))) as ex:
        futs = {n: ex.submit(_run_mutant, n, work) for n in STRENGTH_MUTANTS}
        return {n: f.result() for n, f in futs.items()}


@pytest.mark.parametrize("name", STRENGTH_MUTANTS)
def test_gpu_metrics_reject_planted_mistake(mutant_results, name):
    kind = kind_of(name)
    path = mutant_results[name]
    if path is None:
        print(f"{name}: the mutant oracle refuses to run on these inputs (every case caught)")
        return
    ref = reference(kind)
    missed = []
    with np.load(path, allow_pickle=False) as z:
        for i, c in enumerate(CASES[kind]):
            got = {n.split("/", 1)[1]: z[n] for n in z.files if n.startswith(f"{i}/")}
            rejected, txt = case_rejects(kind, c, got, ref[i])
            print(f"{name} case {i} {c}: {'rejected' if rejected else 'passed'} {txt}")
            if not rejected and (name, i) not in EXEMPT:
                missed.append((i, c))
    assert not missed, f"{name} would pass the GPU metrics on cases {missed}"
