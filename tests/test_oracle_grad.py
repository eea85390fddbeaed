"""Pins of the oracle's gradients (``oracle.gdn_bwd``, ``oracle.polar_bwd``).

The gradients are checked against central finite differences of the oracle's own forward
definitions in fp64 (``gdn_sequential``, ``polar_fwd`` materialised), which are pinned
independently by their own tests.  With a step of 1e-5 the central difference of a smooth
function agrees with the derivative to about 1e-9 relative, so every coordinate of every input
and parameter is compared at 1e-6.  The loss is sum(dO * o) (+ sum(dS * S_T) for the memory), so a
dropped term, a wrong sign, a transposed operand or a wrong index in any gradient fails here.
Cases cover grouped heads (several query heads per kv head), the clamped direction normaliser
(||s|| <= eps) and a non-zero initial memory state.
"""
import numpy as np
import pytest

import oracle

H_FD = 1e-5


def _fd(f, x, h=H_FD):
    """Central differences of the scalar f() with respect to every element of x (in place)."""
    g = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        x0 = x[i]
        x[i] = x0 + h
        fp = f()
        x[i] = x0 - h
        fm = f()
        x[i] = x0
        g[i] = (fp - fm) / (2 * h)
    return g


def _close(a, b, tol=1e-6):
    scale = max(1.0, float(np.max(np.abs(b))))
    err = float(np.max(np.abs(a - b))) / scale
    assert err < tol, err


# ----------------------------------------------------------------------------
# gated-delta memory
# ----------------------------------------------------------------------------
def _gdn_case(seed, B=1, T=6, H=2, Dk=3, Dv=4, init=True):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, T, H, Dk))
    k = rng.standard_normal((B, T, H, Dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, Dv))
    alpha = rng.uniform(0.6, 0.99, (B, T, H))
    beta = rng.uniform(0.1, 0.9, (B, T, H))
    S0 = rng.standard_normal((B, H, Dv, Dk)) * 0.5 if init else None
    dO = rng.standard_normal((B, T, H, Dv))
    dSf = rng.standard_normal((B, H, Dv, Dk))
    return q, k, v, alpha, beta, S0, dO, dSf


@pytest.mark.parametrize("seed,init,final", [(0, True, True), (1, False, True), (2, True, False)])
def test_gdn_grad_matches_finite_differences(seed, init, final):
    q, k, v, alpha, beta, S0, dO, dSf = _gdn_case(seed, init=init)
    if not final:
        dSf = None

    def loss():
        o, fin = oracle.gdn_sequential(q, k, v, alpha, beta, init_state=S0, threads=1)
        val = float(np.sum(o * dO))
        if dSf is not None:
            val += float(np.sum(fin * dSf))
        return val

    g = oracle.gdn_bwd(q, k, v, alpha, beta, dO, init_state=S0, dS_final=dSf, threads=1)
    for name, x in (("dq", q), ("dk", k), ("dv", v), ("dalpha", alpha), ("dbeta", beta)):
        _close(g[name], _fd(loss, x))
    if S0 is not None:
        _close(g["dinit"], _fd(loss, S0))


def test_gdn_grad_single_token_closed_form():
    """One token from state S0, worked by hand: o = S1 q with S1 = a (S0 - b S0 k k^T) + b v k^T,
    so with G = dO q^T: dq = S1^T dO, dv = b G k = b (q . k) dO, dalpha = <G, S0 - b S0 k k^T> and
    the gradient on S0 is a G (I - b k k^T)."""
    rng = np.random.default_rng(5)
    Dk = Dv = 5
    q, k, v = (rng.standard_normal((1, 1, 1, Dk)) for _ in range(3))
    S0 = rng.standard_normal((1, 1, Dv, Dk))
    a, b = np.full((1, 1, 1), 0.8), np.full((1, 1, 1), 0.3)
    dO = rng.standard_normal((1, 1, 1, Dv))
    kk, qq, vv, S, g = k[0, 0, 0], q[0, 0, 0], v[0, 0, 0], S0[0, 0], dO[0, 0, 0]
    S1 = 0.8 * (S - 0.3 * np.outer(S @ kk, kk)) + 0.3 * np.outer(vv, kk)
    r = oracle.gdn_bwd(q, k, v, a, b, dO, init_state=S0, threads=1)
    assert np.allclose(r["dq"][0, 0, 0], S1.T @ g, atol=1e-12)
    assert np.allclose(r["dv"][0, 0, 0], 0.3 * (qq @ kk) * g, atol=1e-12)
    G = np.outer(g, qq)
    assert np.isclose(r["dalpha"][0, 0, 0], np.sum(G * (S - 0.3 * np.outer(S @ kk, kk))), atol=1e-12)
    assert np.allclose(r["dinit"][0, 0], 0.8 * G @ (np.eye(Dk) - 0.3 * np.outer(kk, kk)), atol=1e-12)


def test_gdn_grad_is_linear_in_upstream():
    q, k, v, alpha, beta, S0, dO, dSf = _gdn_case(7, B=2, T=9)
    g1 = oracle.gdn_bwd(q, k, v, alpha, beta, dO, init_state=S0, dS_final=dSf)
    g2 = oracle.gdn_bwd(q, k, v, alpha, beta, 2.5 * dO, init_state=S0, dS_final=2.5 * dSf)
    for n in g1:
        assert np.allclose(g2[n], 2.5 * g1[n], rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------------------
# Polar attention
# ----------------------------------------------------------------------------
def _polar_case(seed, B=1, T=6, Hq=4, Hkv=2, D=4, eps=1e-12):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, T, Hq, D)) * 1.5
    k = rng.standard_normal((B, T, Hkv, D)) * 1.5
    v = rng.standard_normal((B, T, Hkv, D))
    params = {"temp_raw": rng.uniform(-1, 1, Hq), "null_slope_raw": rng.uniform(-1, 1, Hq),
              "null_bias": rng.uniform(-0.5, 1.0, Hq), "mag_beta": rng.uniform(0.2, 1.5, Hq),
              "v_null": rng.standard_normal((Hq, D)) * 0.5, "eps": eps}
    dO = rng.standard_normal((B, T, Hq, D))
    return q, k, v, params, dO


@pytest.mark.parametrize("seed,Hq,Hkv,eps", [(0, 4, 2, 1e-12), (1, 2, 2, 1e-12), (2, 4, 1, 1e-12), (3, 2, 1, 5.0)])
def test_polar_grad_matches_finite_differences(seed, Hq, Hkv, eps):
    q, k, v, params, dO = _polar_case(seed, Hq=Hq, Hkv=Hkv, eps=eps)

    def loss():
        return float(np.sum(oracle.polar_fwd(q, k, v, params, threads=1)["o"] * dO))

    g = oracle.polar_bwd(q, k, v, params, dO, threads=1)
    for name, x in (("dq", q), ("dk", k), ("dv", v)):
        _close(g[name], _fd(loss, x))
    for name in ("temp_raw", "null_slope_raw", "null_bias", "mag_beta", "v_null"):
        _close(g["d_" + name], _fd(loss, params[name]))


def test_polar_grad_clamped_rows_have_no_projection():
    """With eps above every ||s||, o = mu s / eps and the direction gradient is dc / eps: the
    gradient on v then equals the softmax-weighted upstream mu dO / eps summed over rows, which a
    plain numpy evaluation of the materialised weights gives directly when mu does not depend on v."""
    q, k, v, params, dO = _polar_case(4, Hq=1, Hkv=1, eps=50.0)
    g = oracle.polar_bwd(q, k, v, params, dO)
    qq, kk = q[0, :, 0], k[0, :, 0]
    T, D = qq.shape
    a = np.log1p(np.exp(params["temp_raw"][0]))
    sl = np.log1p(np.exp(params["null_slope_raw"][0]))
    dv = np.zeros((T, D))
    for i in range(T):
        n = i + 1
        t = 1 + a * np.log(n)
        nu = params["null_bias"][0] + sl * np.sqrt(np.log(n + 1))
        logits = np.append(t * (kk[:n] @ qq[i]) / np.sqrt(D), t * nu)
        w = np.exp(logits - logits.max())
        w /= w.sum()
        R, Q2 = w[:n].sum(), (w[:n] ** 2).sum()
        mu = np.tanh(params["mag_beta"][0] * np.log1p(R ** 3 / Q2))
        dv[:n] += np.outer(w[:n], mu * dO[0, i, 0] / 50.0)
    assert np.allclose(g["dv"][0, :, 0], dv, atol=1e-12)


def test_polar_grad_single_key_row():
    """A row that sees one key depends on q only through the single logit t (q . k_0) / sqrt(D), so
    its query gradient is a multiple of k_0."""
    q, k, v, params, dO = _polar_case(6, T=1, Hq=1, Hkv=1, D=6)
    g = oracle.polar_bwd(q, k, v, params, dO)
    dq, k0 = g["dq"][0, 0, 0], k[0, 0, 0]
    assert np.allclose(dq - (dq @ k0) / (k0 @ k0) * k0, 0.0, atol=1e-12)


def test_polar_grad_magnitude_sums():
    """The magnitude sums returned beside the scalar parameter gradients bound them (triangle
    inequality) and equal their absolute value when only one row contributes (T = 1)."""
    q, k, v, params, dO = _polar_case(8, Hq=2, Hkv=1)
    g = oracle.polar_bwd(q, k, v, params, dO)
    for n in ("d_temp_raw", "d_null_slope_raw", "d_null_bias", "d_mag_beta"):
        assert np.all(g["abs_" + n] >= np.abs(g[n]) - 1e-15)
    g1 = oracle.polar_bwd(q[:, :1], k[:, :1], v[:, :1], params, dO[:, :1])
    for n in ("d_null_slope_raw", "d_null_bias", "d_mag_beta"):
        assert np.allclose(g1["abs_" + n], np.abs(g1[n]), rtol=1e-12, atol=1e-300)
    # row 0 sees one key and n = 1 (ln n = 0): it adds nothing to the temperature's gradient
    assert g1["abs_d_temp_raw"][0] == 0.0 and g1["d_temp_raw"][0] == 0.0
