"""Pins for the fp64 Polar-attention oracle (CPU only).

Each test checks the oracle against something other than itself:
  * a closed form for a special case (uniform logits, a single key),
  * a reduction to a library routine (``torch.nn.functional.scaled_dot_product_attention``
    in fp64 once the null sink and the temperature are switched off, or scaled per row),
  * the bounded-channel statements of Appendix A.2 (||c|| <= 1, mu in [0, 1),
    participation ratio m for weights uniform over m keys),
  * exact identities: streaming statistics with a segment merge (Appendix C.3, Table 6)
    equal the materialised single softmax (Appendix C.2); decode equals the last row.
Mistakes such as log base 2, n_i = i instead of i + 1, a null logit without the
temperature, a missing 1/sqrt(D), an off-by-one causal mask, a dropped null value or a
missing normalisation each break at least one test.
"""
import math

import numpy as np
import pytest
import torch

import oracle


def _softplus(x):
    return math.log1p(math.exp(x)) if x < 30 else x


def _params(rng, Hq, D, **over):
    p = {
        "temp_raw": np.linspace(-2.0, 1.0, Hq),
        "null_slope_raw": np.linspace(0.0, 2.0, Hq),
        "null_bias": np.linspace(0.0, 1.0, Hq),
        "mag_beta": np.linspace(0.1, 1.0, Hq),
        "v_null": rng.standard_normal((Hq, D)),
        "eps": 1e-12,
    }
    p.update(over)
    return p


def _qkv(rng, B, T, Hq, Hkv, D):
    return (rng.standard_normal((B, T, Hq, D)), rng.standard_normal((B, T, Hkv, D)),
            rng.standard_normal((B, T, Hkv, D)))


def test_uniform_logits_closed_form(rng):
    """q = 0: all n real logits are 0, so the real weights are uniform.  Then n_eff = n,
    real mass R = n / (n + e^{t nu}), m_eff = n R, mu = tanh(beta ln(1 + m_eff)) and the
    direction is normalize(sum_j v_j + e^{t nu} v_null), with t = 1 + softplus(a) ln n and
    nu = b + softplus(g) sqrt(ln(n+1)) (Section 3.2)."""
    B, T, Hq, D = 1, 40, 3, 8
    _, k, v = _qkv(rng, B, T, Hq, Hq, D)
    q = np.zeros((B, T, Hq, D))
    p = _params(rng, Hq, D)
    r = oracle.polar_fwd(q, k, v, p)
    for h in range(Hq):
        a, g = _softplus(p["temp_raw"][h]), _softplus(p["null_slope_raw"][h])
        for i in range(T):
            n = i + 1
            t = 1 + a * math.log(n)
            nu = p["null_bias"][h] + g * math.sqrt(math.log(n + 1))
            e = math.exp(t * nu)
            R = n / (n + e)
            assert r["neff"][0, i, h] == pytest.approx(n, rel=1e-12)
            assert r["meff"][0, i, h] == pytest.approx(n * R, rel=1e-12)
            mu = math.tanh(p["mag_beta"][h] * math.log(1 + n * R))
            assert r["mu"][0, i, h] == pytest.approx(mu, rel=1e-12)
            s = v[0, : i + 1, h].sum(axis=0) + e * p["v_null"][h]
            np.testing.assert_allclose(r["o"][0, i, h], mu * s / np.linalg.norm(s), rtol=1e-11, atol=1e-14)


def test_single_key_closed_form(rng):
    """T = 1: t = 1, R = sigmoid(q.k/sqrt(D) - nu) with nu = b + softplus(g) sqrt(ln 2),
    n_eff = 1, m_eff = R, mu = tanh(beta ln(1+R)), c = normalize(R v_0 + (1-R) v_null)."""
    B, Hq, D = 2, 4, 16
    q, k, v = _qkv(rng, B, 1, Hq, Hq, D)
    p = _params(rng, Hq, D, null_bias=np.array([0.0, 0.3, -0.5, 1.0]))
    r = oracle.polar_fwd(q, k, v, p)
    for b in range(B):
        for h in range(Hq):
            nu = p["null_bias"][h] + _softplus(p["null_slope_raw"][h]) * math.sqrt(math.log(2))
            x = q[b, 0, h] @ k[b, 0, h] / math.sqrt(D)
            R = 1 / (1 + math.exp(-(x - nu)))
            assert r["neff"][b, 0, h] == pytest.approx(1.0, rel=1e-12)
            assert r["meff"][b, 0, h] == pytest.approx(R, rel=1e-12)
            mu = math.tanh(p["mag_beta"][h] * math.log1p(R))
            assert r["mu"][b, 0, h] == pytest.approx(mu, rel=1e-12)
            s = R * v[b, 0, h] + (1 - R) * p["v_null"][h]
            np.testing.assert_allclose(r["o"][b, 0, h], mu * s / np.linalg.norm(s), rtol=1e-11)


def _sdpa_rows(q, k, v, scale_rows):
    """Reference by library: per query row i, softmax(scale_i q_i k_j) over j <= i, via torch SDPA
    (fp64, CPU).  Also returns the weights for the participation ratio."""
    B, T, H, D = q.shape
    out = np.zeros((B, T, H, D))
    pr = np.zeros((B, T, H))
    for i in range(T):
        qi = torch.from_numpy(q[:, i : i + 1]).permute(0, 2, 1, 3)  # [B,H,1,D]
        kk = torch.from_numpy(k[:, : i + 1]).permute(0, 2, 1, 3)
        vv = torch.from_numpy(v[:, : i + 1]).permute(0, 2, 1, 3)
        sc = float(scale_rows[i])
        o = torch.nn.functional.scaled_dot_product_attention(qi, kk, vv, scale=sc)
        out[:, i] = o[:, :, 0].numpy()
        w = torch.softmax(qi @ kk.transpose(-1, -2) * sc, dim=-1)[:, :, 0]  # [B,H,i+1]
        pr[:, i] = (1.0 / (w ** 2).sum(-1)).numpy()
    return out, pr


def test_reduces_to_sdpa_without_null_or_temperature(rng):
    """null_bias -> -1e4 removes the null sink and temp_raw -> -1e4 makes t = 1: the direction
    channel is then normalize(causal SDPA(q, k, v)), n_eff = 1/sum w^2 and m_eff = n_eff."""
    B, T, H, D = 2, 33, 2, 16
    q, k, v = _qkv(rng, B, T, H, H, D)
    p = _params(rng, H, D, null_bias=np.full(H, -1e4), temp_raw=np.full(H, -1e4))
    r = oracle.polar_fwd(q, k, v, p)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q).permute(0, 2, 1, 3), torch.from_numpy(k).permute(0, 2, 1, 3),
        torch.from_numpy(v).permute(0, 2, 1, 3), is_causal=True).permute(0, 2, 1, 3).numpy()
    c = ref / np.linalg.norm(ref, axis=-1, keepdims=True)
    np.testing.assert_allclose(r["o"], r["mu"][..., None] * c, rtol=1e-10, atol=1e-13)
    _, pr = _sdpa_rows(q, k, v, np.full(T, 1 / math.sqrt(D)))
    np.testing.assert_allclose(r["neff"], pr, rtol=1e-10)
    np.testing.assert_allclose(r["meff"], pr, rtol=1e-10)


def test_temperature_scales_real_logits(rng):
    """With the null removed, row i is SDPA with scale t_i / sqrt(D), t_i = 1 + softplus(a) ln(i+1)."""
    B, T, H, D = 1, 30, 3, 8
    q, k, v = _qkv(rng, B, T, H, H, D)
    temp_raw = np.array([-1.0, 0.0, 1.5])
    p = _params(rng, H, D, null_bias=np.full(H, -1e4), temp_raw=temp_raw)
    r = oracle.polar_fwd(q, k, v, p)
    for h in range(H):
        a = _softplus(temp_raw[h])
        scale = np.array([(1 + a * math.log(i + 1)) / math.sqrt(D) for i in range(T)])
        ref, pr = _sdpa_rows(q[:, :, h : h + 1], k[:, :, h : h + 1], v[:, :, h : h + 1], scale)
        c = ref / np.linalg.norm(ref, axis=-1, keepdims=True)
        np.testing.assert_allclose(r["o"][:, :, h], r["mu"][:, :, h, None] * c[:, :, 0], rtol=1e-10, atol=1e-13)
        np.testing.assert_allclose(r["neff"][:, :, h], pr[:, :, 0], rtol=1e-10)


def test_participation_ratio_of_uniform_subset(rng):
    """Appendix A.2: weights uniform over m real keys give participation ratio m.  Keys are
    +-c u with q = u, so m keys share the top logit and the rest are suppressed by e^{-2c t/sqrt(D)}."""
    D, T = 8, 24
    u = np.zeros(D)
    u[0] = 1.0
    sign = -np.ones(T)
    chosen = [0, 3, 4, 10, 17, 23]
    sign[chosen] = 1.0
    c = 300.0
    k = (sign[:, None] * c * u)[None, :, None, :]
    q = np.repeat(u[None, None, None, :], T, axis=1)
    v = rng.standard_normal((1, T, 1, D))
    p = _params(rng, 1, D, null_bias=np.array([-1e4]))
    r = oracle.polar_fwd(q, k, v, p)
    for i in range(T):
        m = sum(1 for j in chosen if j <= i)
        if m == 0:
            continue
        assert r["neff"][0, i, 0] == pytest.approx(m, rel=1e-9)
        want = np.mean([v[0, j, 0] for j in chosen if j <= i], axis=0)
        np.testing.assert_allclose(r["o"][0, i, 0] / r["mu"][0, i, 0], want / np.linalg.norm(want), rtol=1e-9)


def test_bounded_channels(rng):
    """||c|| <= 1 so ||o|| <= mu;  0 <= mu <= 1 (strictly below 1 where the tanh argument is
    moderate);  1 <= n_eff <= n;  0 <= m_eff < n (Appendix A.2)."""
    B, T, Hq, D = 2, 64, 4, 16
    q, k, v = _qkv(rng, B, T, Hq, Hq, D)
    q *= 3.0
    p = _params(rng, Hq, D)
    r = oracle.polar_fwd(q, k, v, p)
    n = np.arange(1, T + 1)[None, :, None]
    on = np.linalg.norm(r["o"], axis=-1)
    np.testing.assert_allclose(on, r["mu"], rtol=1e-12)  # s != 0 here, so ||c|| = 1
    assert np.all(r["mu"] >= 0) and np.all(r["mu"] <= 1)
    arg = p["mag_beta"][None, None, :] * np.log1p(r["meff"])
    assert np.all(r["mu"][arg < 8] < 1)
    assert np.all(r["neff"] >= 1 - 1e-12) and np.all(r["neff"] <= n * (1 + 1e-12))
    assert np.all(r["meff"] >= 0) and np.all(r["meff"] < n)


def test_zero_values_give_zero_output(rng):
    """v = v_null = 0: s_i = 0, the eps clamp keeps c = 0 finite, so o = 0."""
    B, T, H, D = 1, 9, 2, 8
    q, k, _ = _qkv(rng, B, T, H, H, D)
    v = np.zeros((B, T, H, D))
    p = _params(rng, H, D, v_null=np.zeros((H, D)))
    r = oracle.polar_fwd(q, k, v, p)
    assert np.all(r["o"] == 0.0)
    assert np.all(np.isfinite(r["mu"]))


@pytest.mark.parametrize("block,nsplit", [(1, 1), (5, 1), (64, 1), (16, 3), (7, 7), (64, 40)])
def test_streaming_and_split_equal_materialised(rng, block, nsplit):
    """Table 6 streaming (rescale by exp(M_old - M_new), squared accumulator by its square) and
    the merge of key segments reproduce the single materialised softmax."""
    B, T, Hq, Hkv, D = 1, 90, 4, 2, 8
    q, k, v = _qkv(rng, B, T, Hq, Hkv, D)
    q *= 2.0
    p = _params(rng, Hq, D)
    rows = np.array([0, 1, 2, 31, 63, 64, 89])
    a = oracle.polar_fwd(q, k, v, p, rows=rows)
    s = oracle.polar_fwd(q, k, v, p, rows=rows, mode="streaming", block=block, nsplit=nsplit)
    for key in ("o", "mu", "meff", "neff"):
        np.testing.assert_allclose(s[key], a[key], rtol=1e-11, atol=1e-14)


def test_grouped_kv_heads(rng):
    """Query head h reads kv head h // (Hq/Hkv): same result as repeating the kv heads."""
    B, T, Hq, Hkv, D = 1, 20, 6, 2, 8
    q, k, v = _qkv(rng, B, T, Hq, Hkv, D)
    p = _params(rng, Hq, D)
    g = oracle.polar_fwd(q, k, v, p)
    rep = np.repeat(np.arange(Hkv), Hq // Hkv)
    f = oracle.polar_fwd(q, k[:, :, rep], v[:, :, rep], p)
    for key in ("o", "mu", "meff", "neff"):
        np.testing.assert_allclose(g[key], f[key], rtol=0, atol=0)


def test_decode_equals_last_causal_row(rng):
    """Decode over cache slots 0..L-1 equals row L-1 of the causal forward; slots past L are ignored."""
    B, L, Lmax, Hq, Hkv, D = 2, 37, 50, 4, 4, 8
    q, k, v = _qkv(rng, B, Lmax, Hq, Hkv, D)
    p = _params(rng, Hq, D)
    fwd = oracle.polar_fwd(q[:, :L], k[:, :L], v[:, :L], p, rows=[L - 1])
    k2, v2 = k.copy(), v.copy()
    k2[:, L:] = 1e6
    v2[:, L:] = np.nan
    dec = oracle.polar_decode(q[:, L - 1], k2, v2, L, p)
    for key in ("o", "mu", "meff", "neff"):
        np.testing.assert_allclose(dec[key], fwd[key][:, 0], rtol=1e-13, atol=1e-15)


def test_row_sampling_matches_full(rng):
    B, T, H, D = 1, 25, 2, 8
    q, k, v = _qkv(rng, B, T, H, H, D)
    p = _params(rng, H, D)
    full = oracle.polar_fwd(q, k, v, p)
    rows = [24, 0, 7]
    part = oracle.polar_fwd(q, k, v, p, rows=rows)
    for key in ("o", "mu", "meff", "neff"):
        np.testing.assert_array_equal(part[key], full[key][:, rows])
