"""Shared helpers for GPU-vs-oracle parity tests.

Error metric: max |x_gpu - x_oracle| / rms(x_oracle), compared element by element on the
same seeded inputs.  Budgets: 2e-2 for bf16 inputs, 1e-4 for fp32.

Outputs stored in bf16 carry one more unavoidable error: the cast of each element to bf16,
at most half a bf16 ulp.  bf16 keeps 8 significant bits, so half an ulp is at most 2^-8 of the
value (the unit roundoff u; the bound is reached at the bottom of a binade: 1 + 2^-8 rounds to
1, and 2^-9 is only the relative size near the top of one).  Where single elements are several
times larger than the RMS (Polar rows concentrated on a few keys), that cast alone could exceed
2e-2 of the RMS even for the exact result, so bf16-typed outputs are scored with
``rel_err_bf16``: the same metric after allowing each element u = 2^-8 of its own magnitude.

Every metric here also records the plain max |x_gpu - x_oracle| / rms(x_oracle) of the same
comparison (no allowance, no per-row or per-tensor rescaling); ``note`` prints the figures
recorded since its previous call beside the scored ones, so every logged case shows both.
"""
import sys

import numpy as np

TOL = {"bf16": 2e-2, "f32": 1e-4}
BF16_UNIT_ROUNDOFF = 2.0 ** -8  # bound of one round-to-nearest cast to bf16, relative to the value

_PLAIN = []  # plain max-abs / RMS of the comparisons made since the last note()


def _arrays(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    return got, ref


def plain_err(got, ref) -> float:
    """max |got - ref| / rms(ref), with nothing subtracted or rescaled."""
    got, ref = _arrays(got, ref)
    rms = np.sqrt(np.mean(ref ** 2))
    d = float(np.max(np.abs(got - ref))) if got.size else 0.0
    return d / rms if rms > 0 else d


def _record(got, ref):
    _PLAIN.append(plain_err(got, ref))


def to_np(t):
    t = t.detach().cpu()
    if str(t.dtype) in ("torch.bfloat16", "torch.float16"):
        t = t.float()
    return t.double().numpy()


def rel_err(got, ref) -> float:
    got, ref = _arrays(got, ref)
    _record(got, ref)
    rms = np.sqrt(np.mean(ref ** 2))
    if rms == 0:
        return float(np.max(np.abs(got)))
    return float(np.max(np.abs(got - ref)) / rms)


def rel_err_bf16(got, ref) -> float:
    """max(|got - ref| - 2^-8 |ref|, 0) / rms(ref): the RMS budget on top of the output cast."""
    got, ref = _arrays(got, ref)
    _record(got, ref)
    rms = np.sqrt(np.mean(ref ** 2))
    excess = np.maximum(np.abs(got - ref) - BF16_UNIT_ROUNDOFF * np.abs(ref), 0.0)
    return float(np.max(excess) / rms) if rms > 0 else float(np.max(excess))


def rel_err_elem(got, ref) -> float:
    """max |got - ref| / |ref| over elements (denominator floored at 1e-6 rms(ref)).

    For positive quantities with a heavy-tailed spread, such as the effective count
    m_eff (1 up to T): rounding the attention weights to bf16 moves each of them by up
    to 2^-9 of itself, so the error of such a quantity scales with its own value and an
    RMS-normalised metric would charge the largest rows many times over."""
    got, ref = _arrays(got, ref)
    _record(got, ref)
    floor = 1e-6 * max(np.sqrt(np.mean(ref ** 2)), 1e-30)
    return float(np.max(np.abs(got - ref) / np.maximum(np.abs(ref), floor)))


def rel_err_rows_bf16(got, ref, allow=None) -> float:
    """Like rel_err_bf16, but each output row (last axis) is measured against its own RMS.

    For plain softmax attention (the NoPE / RoPE control cores) a row is a convex combination
    of value rows, so its scale shrinks roughly as 1/sqrt(keys seen): the first rows of a
    causal sequence are ~sqrt(T) times the global RMS, and the relative rounding of the bf16
    weights acts on each row's own scale (floor: 1e-3 of the global RMS).  ``allow`` (same
    shape) is a further per-element allowance subtracted before scoring, such as the
    tolerance for a documented rounding of the operands."""
    got, ref = _arrays(got, ref)
    _record(got, ref)
    rms_all = np.sqrt(np.mean(ref ** 2))
    rms_row = np.maximum(np.sqrt(np.mean(ref ** 2, axis=-1, keepdims=True)), 1e-3 * rms_all)
    excess = np.abs(got - ref) - BF16_UNIT_ROUNDOFF * np.abs(ref)
    if allow is not None:
        excess = excess - np.asarray(allow, dtype=np.float64)
    return float(np.max(np.maximum(excess, 0.0) / rms_row))


def out_err(got, ref, dtype: str) -> float:
    """Metric for an output tensor written in ``dtype``."""
    return rel_err_bf16(got, ref) if dtype == "bf16" else rel_err(got, ref)


def note(msg: str) -> None:
    """Print and flush progress so a GPU run names the case it is on; the plain max-abs / RMS
    of every comparison made since the previous note is appended."""
    if _PLAIN:
        msg += "  plain=[" + ", ".join(f"{p:.3e}" for p in _PLAIN) + "]"
        _PLAIN.clear()
    print(msg, flush=True)
    sys.stdout.flush()


def sample_rows(T: int, seed: int = 0, n_random: int = 24, tile: int = 256, chunk: int = 64):
    """Query rows to check at long lengths: first and last rows, rows on both sides of
    query-tile and key-block boundaries, and seeded random rows."""
    rows = set(range(min(T, 8))) | set(range(max(0, T - 8), T))
    for b in (tile, chunk):
        for x in range(b, T, max(b, T // 6 // b * b or b)):
            rows.update({x - 1, x})
    rng = np.random.default_rng(seed)
    rows.update(rng.integers(0, T, size=n_random).tolist())
    return sorted(r for r in rows if 0 <= r < T)


def rel_err_max(got, ref) -> float:
    """max |got - ref| / max |ref|: the error against the tensor's own scale.

    For gradients, whose elements are heavy-tailed (the largest 10-20 times the RMS) and each a
    sum whose terms are set by the largest products of its row, bf16 arithmetic leaves an absolute
    error proportional to that scale; an RMS-normalised maximum would charge it 10-20 times."""
    got, ref = _arrays(got, ref)
    _record(got, ref)
    m = float(np.max(np.abs(ref)))
    return float(np.max(np.abs(got - ref))) / m if m > 0 else float(np.max(np.abs(got)))


def rel_err_fro(got, ref) -> float:
    """||got - ref||_F / ||ref||_F."""
    got, ref = _arrays(got, ref)
    _record(got, ref)
    n = float(np.linalg.norm(ref))
    return float(np.linalg.norm(got - ref)) / n if n > 0 else float(np.linalg.norm(got))


# ---- gradient scoring shared by the backward GPU tests and the metric-strength test ----------
POLAR_GRADS = ("dq", "dk", "dv", "d_temp_raw", "d_null_slope_raw", "d_null_bias", "d_mag_beta", "d_v_null")
POLAR_SCALAR_PARAMS = ("d_temp_raw", "d_null_slope_raw", "d_null_bias", "d_mag_beta")
POLAR_BWD_TOL_MAX, POLAR_BWD_TOL_FRO = 2e-2, 1e-2
GDN_GRADS = ("dq", "dk", "dv", "dalpha", "dbeta", "dinit")


def sum_err(got, ref, mag) -> float:
    """max over heads of |gpu - oracle| / (sum of the magnitudes of its terms): a parameter
    gradient is a sum over all B T rows whose terms cancel (by 15-20 times on these inputs), and
    its rounding error scales with the magnitude of the terms, not with the sum.  For the
    temperature each row's term is itself a sum over keys of bf16-rounded logit gradients times
    q.k, taken term by term."""
    got, ref = _arrays(got, ref)
    _record(got, ref)
    return float(np.max(np.abs(got - ref) / np.maximum(np.asarray(mag, dtype=np.float64), 1e-30)))


def polar_grad_errors(got: dict, ref: dict, names=POLAR_GRADS) -> dict:
    """{name: (max measure, Frobenius measure)} of Polar gradients (numpy arrays) against the
    oracle's; the four scalar parameter gradients by sum_err for both."""
    out = {}
    for n in names:
        if n in POLAR_SCALAR_PARAMS:
            e = sum_err(got[n], ref[n], ref["abs_" + n])
            out[n] = (e, e)
        else:
            out[n] = (rel_err_max(got[n], ref[n]), rel_err_fro(got[n], ref[n]))
    return out


def polar_grad_failures(errs: dict) -> dict:
    return {n: e for n, e in errs.items() if not (e[0] <= POLAR_BWD_TOL_MAX and e[1] <= POLAR_BWD_TOL_FRO)}


def gdn_grad_tol(name: str, dtype: str) -> float:
    """Budget of one memory gradient: 1e-4 of the top scale for fp32-stored outputs; the bf16
    storage of dq, dk, dv (2^-9 of an element) gets 4e-3."""
    return 4e-3 if (dtype == "bf16" and name in ("dq", "dk", "dv")) else 1e-4


def gdn_grad_errors(got: dict, ref: dict, names=GDN_GRADS) -> dict:
    return {n: (rel_err_max(got[n], ref[n]), rel_err_fro(got[n], ref[n])) for n in names}


def gdn_grad_failures(errs: dict, dtype: str) -> dict:
    return {n: e for n, e in errs.items() if not (e[0] <= gdn_grad_tol(n, dtype) and e[1] <= gdn_grad_tol(n, dtype))}
