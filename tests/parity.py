"""Shared helpers for GPU-vs-oracle parity tests.

Error metric: max |x_gpu - x_oracle| / rms(x_oracle), compared element by element on the
same seeded inputs.  Budgets: 2e-2 for bf16 inputs, 1e-4 for fp32.

Outputs stored in bf16 carry one more unavoidable error: the cast of each element to bf16
(relative half-ulp 2^-9, one ulp 2^-8).  Where single elements are several times larger
than the RMS (Polar rows concentrated on a few keys), that cast alone exceeds 2e-2 of the
RMS even for the exact result, so bf16-typed outputs are scored with ``rel_err_bf16``:
the same metric after allowing each element one bf16 ulp of its own magnitude.
"""
import sys

import numpy as np

TOL = {"bf16": 2e-2, "f32": 1e-4}


def to_np(t):
    t = t.detach().cpu()
    if str(t.dtype) in ("torch.bfloat16", "torch.float16"):
        t = t.float()
    return t.double().numpy()


def rel_err(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    rms = np.sqrt(np.mean(ref ** 2))
    if rms == 0:
        return float(np.max(np.abs(got)))
    return float(np.max(np.abs(got - ref)) / rms)


def rel_err_bf16(got, ref) -> float:
    """max(|got - ref| - 2^-8 |ref|, 0) / rms(ref): the RMS budget on top of the output cast."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    rms = np.sqrt(np.mean(ref ** 2))
    excess = np.maximum(np.abs(got - ref) - 2.0 ** -8 * np.abs(ref), 0.0)
    return float(np.max(excess) / rms) if rms > 0 else float(np.max(excess))


def rel_err_elem(got, ref) -> float:
    """max |got - ref| / |ref| over elements (denominator floored at 1e-6 rms(ref)).

    For positive quantities with a heavy-tailed spread, such as the effective count
    m_eff (1 up to T): rounding the attention weights to bf16 moves each of them by up
    to 2^-9 of itself, so the error of such a quantity scales with its own value and an
    RMS-normalised metric would charge the largest rows many times over."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    floor = 1e-6 * max(np.sqrt(np.mean(ref ** 2)), 1e-30)
    return float(np.max(np.abs(got - ref) / np.maximum(np.abs(ref), floor)))


def rel_err_rows_bf16(got, ref) -> float:
    """Like rel_err_bf16, but each output row (last axis) is measured against its own RMS.

    For plain softmax attention (the NoPE / RoPE control cores) a row is a convex combination
    of value rows, so its scale shrinks roughly as 1/sqrt(keys seen): the first rows of a
    causal sequence are ~sqrt(T) times the global RMS, and the relative rounding of the bf16
    weights acts on each row's own scale (floor: 1e-3 of the global RMS)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    rms_all = np.sqrt(np.mean(ref ** 2))
    rms_row = np.maximum(np.sqrt(np.mean(ref ** 2, axis=-1, keepdims=True)), 1e-3 * rms_all)
    excess = np.maximum(np.abs(got - ref) - 2.0 ** -8 * np.abs(ref), 0.0)
    return float(np.max(excess / rms_row))


def out_err(got, ref, dtype: str) -> float:
    """Metric for an output tensor written in ``dtype``."""
    return rel_err_bf16(got, ref) if dtype == "bf16" else rel_err(got, ref)


def note(msg: str) -> None:
    """Print and flush progress so a GPU run names the case it is on."""
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
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    m = float(np.max(np.abs(ref)))
    return float(np.max(np.abs(got - ref))) / m if m > 0 else float(np.max(np.abs(got)))


def rel_err_fro(got, ref) -> float:
    """||got - ref||_F / ||ref||_F."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    n = float(np.linalg.norm(ref))
    return float(np.linalg.norm(got - ref)) / n if n > 0 else float(np.linalg.norm(got))
