"""The oracle pins are strong enough to catch plausible mistakes in the oracle.

Each case copies ``oracle/oracle.c``, plants one mistake by text substitution, builds
the copy with gcc in a temporary directory, and runs the oracle pin tests against it
(``ATMA_ORACLE_LIB`` points the wrapper at the copy).  Every mutant must fail at least
one pin.  CPU only; the real oracle is untouched.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

MUTANTS = {
    "gdn_erase_sign": ("S[r * Dk + j] - be * u[r] * kt[j]", "S[r * Dk + j] + be * u[r] * kt[j]"),
    "gdn_decay_first_term_only": ("a * (S[r * Dk + j] - be * u[r] * kt[j])", "(a * S[r * Dk + j] - be * u[r] * kt[j])"),
    "gdn_write_transposed": ("S[r * Dk + j] - be * u[r] * kt[j]) + be * vt[r] * kt[j]",
                             "S[r * Dk + j] - be * u[r] * kt[j]) + be * vt[j % Dv] * kt[r % Dk]"),
    "gdn_output_from_old_key": ("for (int j = 0; j < Dk; ++j) s += S[r * Dk + j] * qt[j];",
                                "for (int j = 0; j < Dk; ++j) s += S[r * Dk + j] * kt[j];"),
    "gdn_chunk_decay_sign": ("val = c->beta[TOK(t0 + r)] * exp(g[r] - g[s]) * d;",
                             "val = c->beta[TOK(t0 + r)] * exp(g[s] - g[r]) * d;"),
    "polar_temp_log2": ("const double t = 1.0 + a * log((double)n);                          /* Section 3.2: t_i */",
                        "const double t = 1.0 + a * log2((double)n);"),
    "polar_n_off_by_one": ("const double nu = P->null_bias[h] + s * sqrt(log((double)n + 1.0)); /* Section 3.2: nu_i */",
                           "const double nu = P->null_bias[h] + s * sqrt(log((double)n + 2.0));"),
    "polar_null_without_temperature": ("const double lnull = t * nu;                                        /* virtual null logit */",
                                       "const double lnull = nu;"),
    "polar_no_sqrt_d": ("w[j] = t * d * inv_sqrt_d;", "w[j] = t * d;"),
    "polar_neff_linear": ("const double ne = R * R / Q2;", "const double ne = R / Q2;"),
    "polar_meff_no_mass": ("const double me = ne * R;", "const double me = ne;"),
    "polar_mu_log": ("const double muv = tanh(P->mag_beta[h] * log1p(me));\n    /* direction",
                     "const double muv = tanh(P->mag_beta[h] * log(me));\n    /* direction"),
    "polar_drop_null_value": ("double acc = wnull * P->v_null[(size_t)h * D + x];", "double acc = 0.0;"),
    "polar_no_normalise": ("for (int x = 0; x < D; ++x) o[x] = muv * (o[x] / den);\n    *mu = muv; *meff = me; *neff = ne;\n}\n\n/* Streaming",
                           "for (int x = 0; x < D; ++x) o[x] = muv * o[x];\n    *mu = muv; *meff = me; *neff = ne;\n}\n\n/* Streaming"),
    "polar_causal_off_by_one": ("polar_row_materialised(qi, K, V, stride, stride, i + 1,",
                                "polar_row_materialised(qi, K, V, stride, stride, (i + 2 <= c->T ? i + 2 : i + 1),"),
    "streaming_q2_rho_linear": ("L *= rho; Q2 *= rho * rho;", "L *= rho; Q2 *= rho;"),
    "rope_reflect": ("x[2 * p + 1] = a * s + b * c;", "x[2 * p + 1] = -a * s + b * c;"),
    "rope_half_frequency": ("pos * pow(theta, -2.0 * p / D);", "pos * pow(theta, -1.0 * p / D);"),
    "softmax_no_scale": ("w[j] = d * scale;", "w[j] = d;"),
    "softmax_sees_next_key": ("softmax_row(qi, K, V, D, (size_t)c->Hkv * D, (long)i + 1, D, oi, w);",
                              "softmax_row(qi, K, V, D, (size_t)c->Hkv * D, (long)(i + 1 < T ? i + 2 : i + 1), D, oi, w);"),
    "tolerance_drops_query_term": ("tol[x] = lambda * u * sqrt((sa + sb[x]) / (double)D);",
                                   "tol[x] = lambda * u * sqrt(sb[x] / (double)D);"),
    "tolerance_no_sqrt_d": ("tol[x] = lambda * u * sqrt((sa + sb[x]) / (double)D);",
                            "tol[x] = lambda * u * sqrt(sa + sb[x]);"),
    "tolerance_unnormalised_weights": ("const double wj = w[j] / z;", "const double wj = w[j];"),
    "canon_anticausal": ("const long s = t - j;", "const long s = t + j < T ? t + j : t - j;"),
    "canon_state_offset": ("xv = state[((size_t)b * (K - 1) + (K - 1 + s)) * C + c];",
                           "xv = state[((size_t)b * (K - 1) + (K - 2 + s >= 0 ? K - 2 + s : 0)) * C + c];"),
    "canon_norm_squared": ("yt[h * D + e] /= den;", "yt[h * D + e] /= den * den;"),
    "softmax_decode_query_position": ("rope_vec(qi, D, (double)(cache_len - 1), theta);",
                                      "rope_vec(qi, D, (double)cache_len, theta);"),
    "gdn_bwd_beta_sign": ("db += Gk[r] * (vt[r] - a * u[r]);", "db += Gk[r] * (vt[r] + a * u[r]);"),
    "gdn_bwd_no_decay_of_state_grad": ("G[r * Dk + j] = a * (G[r * Dk + j] - be * Gk[r] * kt[j]);",
                                       "G[r * Dk + j] = (G[r * Dk + j] - be * Gk[r] * kt[j]);"),
    "gdn_bwd_dk_drops_term": ("dkt[j] = be * gv - a * be * (sg + gu);", "dkt[j] = be * gv - a * be * sg;"),
    "gdn_bwd_dq_old_state": ("for (int r = 0; r < Dv; ++r) s += St[r * Dk + j] * gt[r];",
                             "for (int r = 0; r < Dv; ++r) s += Sp[r * Dk + j] * gt[r];"),
    "polar_bwd_no_q2_term": ("const double dwj = dR + 2.0 * w[j] * dQ2 + dv;", "const double dwj = dR + dv;"),
    "polar_bwd_no_projection": ("ds[x] = (mu * g[x] - (clamped ? 0.0 : (s[x] / den) * cdc)) / den;",
                                "ds[x] = mu * g[x] / den;"),
    "polar_bwd_null_temperature": ("dt += dl0 * nu;", "dt += 0.0 * nu;"),
    "polar_bwd_softplus_not_sigmoid": ("dpar[0] += dt * log((double)n) * sigmoid(P->temp_raw[h]);",
                                       "dpar[0] += dt * log((double)n) * softplus(P->temp_raw[h]);"),
    "polar_bwd_meff_power": ("const double dR = dme * 3.0 * R * R / Q2;", "const double dR = dme * 2.0 * R * R / Q2;"),
}


def _run_pins(name, workdir):
    """Builds the mutant and runs every pin against it; returns (exit status, output tail)."""
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    d = workdir / name
    d.mkdir()
    mutated = d / "oracle_mut.c"
    mutated.write_text(src.replace(old, new))
    lib = d / "liboracle_mut.so"
    subprocess.run(["gcc", "-O2", "-std=c99", "-fPIC", "-D_POSIX_C_SOURCE=200809L", "-shared", "-o", str(lib),
                    str(mutated), "-lm", "-lpthread"], check=True)
    env = dict(os.environ, ATMA_ORACLE_LIB=str(lib))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_gdn.py"),
                        os.path.join(ROOT, "tests", "test_oracle_polar.py"),
                        os.path.join(ROOT, "tests", "test_oracle_baseline.py"),
                        os.path.join(ROOT, "tests", "test_oracle_canon.py"),
                        os.path.join(ROOT, "tests", "test_oracle_grad.py")],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=900)
    return r.returncode, r.stdout[-2000:]


@pytest.fixture(scope="module")
def pin_results(tmp_path_factory):
    """Every mutant built and run against the pins up front, one process per CPU (at most 8)."""
    import concurrent.futures as cf

    work = tmp_path_factory.mktemp("mutants")
    with cf.ThreadPoolExecutor(max_workers=max(1, min(8, os.cpu_count() or 1))) as ex:
        futs = {n: ex.submit(_run_pins, n, work) for n in sorted(MUTANTS)}
        return {n: f.result() for n, f in futs.items()}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(pin_results, name):
    rc, out = pin_results[name]
    assert rc != 0, f"mutant {name} survived every pin:\n{out}"
