"""fp64 CPU oracle for the ATMA hot path (gated-delta memory and Polar attention).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  The product library never imports, links
or executes anything in this directory, and this module imports nothing from the
product package.  Inputs of any float precision are widened exactly to fp64;
results are fp64 numpy arrays.

The arithmetic lives in ``oracle.c`` (plain loops, one function per definition);
this module only marshals arrays.  Definitions, by source passage (ATMA paper,
arXiv 2606.25156):

* ``gdn_sequential``  - Section 3.3 equation, run token by token.
* ``gdn_chunked``     - the exact chunked rewrite of the same recurrence
                         (UT transform of the intra-chunk system).
* ``polar_fwd``       - Section 3.2 (t_i, nu_i), Appendix C.2 (one softmax over
                         masked real logits + virtual null logit), Appendix A.2
                         (direction and magnitude channels); ``mode="streaming"``
                         follows Appendix C.3 / Table 6 with a segment merge.
* ``polar_decode``    - the last causal row for a KV cache of ``cache_len`` slots.
* ``rope``, ``softmax_attn``, ``softmax_decode`` - the NoPE / RoPE control cores the
                         paper compares Polar against (Section 3.1): causal softmax
                         attention with scale 1/sqrt(D), optionally after rotating
                         adjacent pairs of q and k by position * theta^(-2p/D).
* ``canon``           - the Canon prologue (Section 3.1): depthwise causal convolution
                         over tokens, optional residual, optional unit L2 norm per head.
* ``gdn_bwd``, ``polar_bwd`` - gradients of a loss through ``gdn_sequential`` and
                         ``polar_fwd`` (the chain rule on the same definitions, in reverse;
                         the paper's materialised path is its gradient reference too,
                         Appendix C.2).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
# A test may point the wrapper at another build of oracle.c (e.g. one with a planted
# mistake, to show that the pins catch it).
_LIB_OVERRIDE = os.environ.get("ATMA_ORACLE_LIB")
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_i64p = ctypes.POINTER(ctypes.c_int64)


def build(force: bool = False) -> str:
    """Compile ``oracle.c`` with gcc (``make -C oracle``)."""
    cmd = ["make", "-C", _HERE] + (["-B"] if force else [])
    subprocess.run(cmd, check=True, stdout=subprocess.DEVNULL)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            _lib = _declare(ctypes.CDLL(_LIB_OVERRIDE))
            return _lib
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(
            os.path.join(_HERE, "oracle.c")
        ):
            build()
        _lib = _declare(ctypes.CDLL(_LIB_PATH))
    return _lib


def _declare(lib):
    i, l, d = ctypes.c_int, ctypes.c_long, ctypes.c_double
    lib.oracle_gdn_sequential.argtypes = [i, i, i, i, i] + [_dp] * 6 + [_dp, _dp, _dp, i]
    lib.oracle_gdn_chunked.argtypes = [i, i, i, i, i, i] + [_dp] * 6 + [_dp, _dp, i]
    lib.oracle_polar_fwd.argtypes = (
        [i, i, i, i, i] + [_dp] * 3 + [_dp] * 5 + [d, _i64p, l, i, l, i] + [_dp] * 4 + [i]
    )
    lib.oracle_polar_decode.argtypes = [i, i, i, i, l, l] + [_dp] * 3 + [_dp] * 5 + [d] + [_dp] * 4 + [i]
    lib.oracle_threads_used.argtypes = [i, l]
    lib.oracle_rope.argtypes = [i, i, i, i, l, d, i, _dp, _dp]
    lib.oracle_softmax_attn.argtypes = [i, i, i, i, i, d, _dp, _dp, _dp, _dp, _dp, d, i]
    lib.oracle_softmax_decode.argtypes = [i, i, i, i, l, l, d, _dp, _dp, _dp, _dp]
    lib.oracle_canon.argtypes = [i, i, i, i, i, i, d, _dp, _dp, _dp, _dp]
    lib.oracle_gdn_bwd.argtypes = [i, i, i, i, i] + [_dp] * 6 + [_dp, _dp] + [_dp] * 6 + [i]
    lib.oracle_polar_bwd.argtypes = [i, i, i, i, i] + [_dp] * 3 + [_dp] * 5 + [d, _dp] + [_dp] * 9 + [i]
    for f in ("oracle_gdn_sequential", "oracle_gdn_chunked", "oracle_polar_fwd", "oracle_polar_decode",
              "oracle_threads_used", "oracle_rope", "oracle_softmax_attn", "oracle_softmax_decode", "oracle_canon",
              "oracle_gdn_bwd", "oracle_polar_bwd"):
        getattr(lib, f).restype = ctypes.c_int
    return lib


def _f64(x) -> np.ndarray:
    """Widen a numpy array or torch CPU tensor (any float dtype) exactly to contiguous fp64."""
    if hasattr(x, "detach"):  # torch tensor
        x = x.detach().to("cpu")
        if str(x.dtype) in ("torch.bfloat16", "torch.float16"):
            x = x.float()
        x = x.double().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(_dp)


def threads_used(nthreads: int, ntasks: int) -> int:
    """Threads the oracle runs for ``ntasks`` independent tasks (0 = one per online core)."""
    return _load().oracle_threads_used(int(nthreads), int(ntasks))


# ----------------------------------------------------------------------------
# gated-delta memory
# ----------------------------------------------------------------------------
def _gdn_args(q, k, v, alpha, beta, init_state):
    q, k, v, alpha, beta = (_f64(x) for x in (q, k, v, alpha, beta))
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    assert k.shape == (B, T, H, Dk) and v.shape == (B, T, H, Dv), (q.shape, k.shape, v.shape)
    assert alpha.shape == (B, T, H) and beta.shape == (B, T, H)
    init = None if init_state is None else _f64(init_state)
    if init is not None:
        assert init.shape == (B, H, Dv, Dk)
    return q, k, v, alpha, beta, init, (B, T, H, Dk, Dv)


def gdn_sequential(q, k, v, alpha, beta, init_state=None, want_states=False, threads=0):
    """Token-by-token recurrence.  Returns (o [B,T,H,Dv], S_T [B,H,Dv,Dk][, S_t history])."""
    q, k, v, alpha, beta, init, (B, T, H, Dk, Dv) = _gdn_args(q, k, v, alpha, beta, init_state)
    o = np.zeros((B, T, H, Dv))
    fin = np.zeros((B, H, Dv, Dk))
    states = np.zeros((B, T, H, Dv, Dk)) if want_states else None
    rc = _load().oracle_gdn_sequential(B, T, H, Dk, Dv, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                       _ptr(init), _ptr(o), _ptr(fin), _ptr(states), int(threads))
    assert rc == 0
    return (o, fin, states) if want_states else (o, fin)


def gdn_chunked(q, k, v, alpha, beta, init_state=None, chunk=64, threads=0):
    """Chunked evaluation of the same recurrence.  Returns (o, S_T)."""
    q, k, v, alpha, beta, init, (B, T, H, Dk, Dv) = _gdn_args(q, k, v, alpha, beta, init_state)
    o = np.zeros((B, T, H, Dv))
    fin = np.zeros((B, H, Dv, Dk))
    rc = _load().oracle_gdn_chunked(B, T, H, Dk, Dv, int(chunk), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                                    _ptr(beta), _ptr(init), _ptr(o), _ptr(fin), int(threads))
    assert rc == 0
    return o, fin


def gdn_decode_step(q, k, v, alpha, beta, state, threads=0):
    """One recurrence step: q,k [B,H,Dk], v [B,H,Dv], alpha,beta [B,H], state [B,H,Dv,Dk].
    Returns (o [B,H,Dv], new_state)."""
    o, fin = gdn_sequential(_f64(q)[:, None], _f64(k)[:, None], _f64(v)[:, None], _f64(alpha)[:, None],
                            _f64(beta)[:, None], init_state=state, threads=threads)
    return o[:, 0], fin


# ----------------------------------------------------------------------------
# Polar attention
# ----------------------------------------------------------------------------
def _params(params, Hq, D):
    out = {}
    for name in ("temp_raw", "null_slope_raw", "null_bias", "mag_beta"):
        out[name] = _f64(params[name]).reshape(Hq)
    out["v_null"] = _f64(params["v_null"]).reshape(Hq, D)
    out["eps"] = float(params.get("eps", 1e-12))
    return out


def polar_fwd(q, k, v, params, rows=None, mode="materialised", block=64, nsplit=1, threads=0):
    """Causal Polar attention for query ``rows`` (default: all).

    q [B,T,Hq,D], k/v [B,T,Hkv,D].  Returns dict with o [B,R,Hq,D] and mu, meff, neff [B,R,Hq]
    (R = len(rows) or T)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, T, Hq, D = q.shape
    Hkv = k.shape[2]
    assert k.shape == (B, T, Hkv, D) and v.shape == (B, T, Hkv, D)
    p = _params(params, Hq, D)
    r = None if rows is None else np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    R = T if r is None else len(r)
    o = np.zeros((B, R, Hq, D))
    mu, meff, neff = (np.zeros((B, R, Hq)) for _ in range(3))
    m = {"materialised": 0, "streaming": 1}[mode]
    rc = _load().oracle_polar_fwd(
        B, T, Hq, Hkv, D, _ptr(q), _ptr(k), _ptr(v), _ptr(p["temp_raw"]), _ptr(p["null_slope_raw"]),
        _ptr(p["null_bias"]), _ptr(p["mag_beta"]), _ptr(p["v_null"]), p["eps"],
        None if r is None else r.ctypes.data_as(_i64p), R, m, int(block), int(nsplit),
        _ptr(o), _ptr(mu), _ptr(meff), _ptr(neff), int(threads))
    assert rc == 0
    return {"o": o, "mu": mu, "meff": meff, "neff": neff}


def polar_decode(q, k_cache, v_cache, cache_len, params, threads=0):
    """q [B,Hq,D], caches [B,Lmax,Hkv,D].  Returns dict o [B,Hq,D], mu/meff/neff [B,Hq]."""
    q, kc, vc = _f64(q), _f64(k_cache), _f64(v_cache)
    B, Hq, D = q.shape
    Lmax, Hkv = kc.shape[1], kc.shape[2]
    p = _params(params, Hq, D)
    o = np.zeros((B, Hq, D))
    mu, meff, neff = (np.zeros((B, Hq)) for _ in range(3))
    rc = _load().oracle_polar_decode(
        B, Hq, Hkv, D, int(cache_len), Lmax, _ptr(q), _ptr(kc), _ptr(vc), _ptr(p["temp_raw"]),
        _ptr(p["null_slope_raw"]), _ptr(p["null_bias"]), _ptr(p["mag_beta"]), _ptr(p["v_null"]), p["eps"],
        _ptr(o), _ptr(mu), _ptr(meff), _ptr(neff), int(threads))
    assert rc == 0
    return {"o": o, "mu": mu, "meff": meff, "neff": neff}


def rope(x, theta=10000.0, pos0=0, bf16=False):
    """x [B,T,H,D]; row t rotated to position pos0 + t (adjacent pairs), rounded to bf16 values
    when ``bf16``.  Returns fp64."""
    x = _f64(x)
    B, T, H, D = x.shape
    y = np.empty_like(x)
    assert _load().oracle_rope(B, T, H, D, int(pos0), float(theta), int(bf16), _ptr(x), _ptr(y)) == 0
    return y


def softmax_attn(q, k, v, rope_theta=0.0, tol_lambda=None, threads=0):
    """Causal softmax attention (NoPE; RoPE with the exact rotation when rope_theta > 0).
    q [B,T,Hq,D], k/v [B,T,Hkv,D].  Returns o [B,T,Hq,D]; with ``tol_lambda`` also, per output
    element, the probabilistic tolerance (Hoeffding, ``tol_lambda`` standard deviations of the
    first-order effect; see oracle.c) for rounding each element of the rotated q and k to the
    nearest bf16 value."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, T, Hq, D = q.shape
    Hkv = k.shape[2]
    assert k.shape == (B, T, Hkv, D) and v.shape == (B, T, Hkv, D)
    o = np.zeros((B, T, Hq, D))
    tol = np.zeros((B, T, Hq, D)) if tol_lambda is not None else None
    assert _load().oracle_softmax_attn(B, T, Hq, Hkv, D, float(rope_theta), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                       _ptr(tol), float(tol_lambda or 0.0), int(threads)) == 0
    return (o, tol) if tol_lambda is not None else o


def softmax_decode(q, k_cache, v_cache, cache_len, rope_theta=0.0):
    """q [B,Hq,D], caches [B,Lmax,Hkv,D] used as given; for RoPE (rope_theta > 0) the cache holds
    keys already rotated to their slot positions and only the query is rotated.  Returns o [B,Hq,D]."""
    q, kc, vc = _f64(q), _f64(k_cache), _f64(v_cache)
    B, Hq, D = q.shape
    Lmax, Hkv = kc.shape[1], kc.shape[2]
    o = np.zeros((B, Hq, D))
    assert _load().oracle_softmax_decode(B, Hq, Hkv, D, int(cache_len), Lmax, float(rope_theta), _ptr(q), _ptr(kc),
                                         _ptr(vc), _ptr(o)) == 0
    return o


def canon(x, w, state=None, residual=False, heads=0, eps=1e-6):
    """x [B,T,C]; w [K,C]; state [B,K-1,C] (previous inputs, oldest first) or None.
    Returns y [B,T,C] (fp64): depthwise causal convolution (+ x when ``residual``), then unit
    L2 norm of each of ``heads`` channel groups when heads > 0."""
    x, w = _f64(x), _f64(w)
    B, T, C = x.shape
    K = w.shape[0]
    st = None if state is None else _f64(state)
    y = np.zeros((B, T, C))
    assert _load().oracle_canon(B, T, C, K, int(bool(residual)), int(heads), float(eps), _ptr(x), _ptr(w), _ptr(st),
                                _ptr(y)) == 0
    return y


# ----------------------------------------------------------------------------
# gradients
# ----------------------------------------------------------------------------
def gdn_bwd(q, k, v, alpha, beta, do, init_state=None, dS_final=None, threads=0):
    """Gradients through the token-by-token memory recurrence for upstream dO [B,T,H,Dv] (and
    dS_final [B,H,Dv,Dk] on the final state, or None).  Returns dict dq, dk, dv, dalpha, dbeta,
    dinit (the gradient on the initial state)."""
    q, k, v, alpha, beta, init, (B, T, H, Dk, Dv) = _gdn_args(q, k, v, alpha, beta, init_state)
    g = _f64(do)
    assert g.shape == (B, T, H, Dv)
    dsf = None if dS_final is None else _f64(dS_final)
    out = {"dq": np.zeros((B, T, H, Dk)), "dk": np.zeros((B, T, H, Dk)), "dv": np.zeros((B, T, H, Dv)),
           "dalpha": np.zeros((B, T, H)), "dbeta": np.zeros((B, T, H)), "dinit": np.zeros((B, H, Dv, Dk))}
    rc = _load().oracle_gdn_bwd(B, T, H, Dk, Dv, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(init),
                                _ptr(g), _ptr(dsf), _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]),
                                _ptr(out["dalpha"]), _ptr(out["dbeta"]), _ptr(out["dinit"]), int(threads))
    assert rc == 0
    return out


def polar_bwd(q, k, v, params, do, threads=0):
    """Gradients of causal Polar attention (materialised form) for upstream dO [B,T,Hq,D].
    Returns dict dq, dk, dv and d_temp_raw, d_null_slope_raw, d_null_bias, d_mag_beta [Hq],
    d_v_null [Hq, D]; also abs_<name> [Hq] for the four scalar parameters: the sum over rows of
    the magnitudes of their per-row contributions (the natural error scale of those sums)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, T, Hq, D = q.shape
    Hkv = k.shape[2]
    assert k.shape == (B, T, Hkv, D) and v.shape == (B, T, Hkv, D)
    g = _f64(do)
    assert g.shape == q.shape
    p = _params(params, Hq, D)
    out = {"dq": np.zeros_like(q), "dk": np.zeros_like(k), "dv": np.zeros_like(v)}
    for n in ("d_temp_raw", "d_null_slope_raw", "d_null_bias", "d_mag_beta"):
        out[n] = np.zeros(Hq)
    out["d_v_null"] = np.zeros((Hq, D))
    absum = np.zeros((4, Hq))
    rc = _load().oracle_polar_bwd(
        B, T, Hq, Hkv, D, _ptr(q), _ptr(k), _ptr(v), _ptr(p["temp_raw"]), _ptr(p["null_slope_raw"]),
        _ptr(p["null_bias"]), _ptr(p["mag_beta"]), _ptr(p["v_null"]), p["eps"], _ptr(g), _ptr(out["dq"]),
        _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["d_temp_raw"]), _ptr(out["d_null_slope_raw"]),
        _ptr(out["d_null_bias"]), _ptr(out["d_mag_beta"]), _ptr(out["d_v_null"]), _ptr(absum), int(threads))
    assert rc == 0
    # scale of each scalar parameter gradient as a sum over rows: sum of the rows' magnitudes
    for e, n in enumerate(("d_temp_raw", "d_null_slope_raw", "d_null_bias", "d_mag_beta")):
        out["abs_" + n] = absum[e]
    return out
