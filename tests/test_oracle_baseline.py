"""Pins of the oracle's NoPE / RoPE control cores (the matched baselines of the ATMA paper,
Section 3.1), checked against what mathematics and a library routine fix:

* NoPE equals torch's scaled-dot-product attention (causal, fp64) with kv heads repeated;
* RoPE rotates each adjacent pair: a D=2 unit vector at position m becomes (cos m, sin m);
  pair norms are preserved; pair p turns by theta^(-2p/D) per position (the textbook
  frequencies); scores depend only on the position difference (shift invariance);
* the decode row equals the last row of the causal forward, with and without RoPE (the decode
  cache holding keys already rotated to their slots);
* identical keys give the plain mean of the values;
* the probabilistic tolerance for rounding the rotated q and k to bf16 (7 standard deviations of
  the first-order effect) covers the actual rounding and random perturbations of the same size,
  is zero where no rounding can matter, and is not vacuous: the actual rounding reaches a fixed
  share of it, and it scales with the rounding unit.
"""
import math

import numpy as np
import pytest
import torch

import oracle


def _sdpa(q, k, v):
    """torch SDPA in fp64 on [B,T,H,D] arrays, causal, kv heads repeated for GQA."""
    Hq, Hkv = q.shape[2], k.shape[2]
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(x)).permute(0, 2, 1, 3) for x in (q, k, v))
    tk = tk.repeat_interleave(Hq // Hkv, dim=1)
    tv = tv.repeat_interleave(Hq // Hkv, dim=1)
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True)
    return o.permute(0, 2, 1, 3).numpy()


@pytest.mark.parametrize("B,T,Hq,Hkv,D", [(1, 1, 1, 1, 8), (2, 37, 4, 2, 16), (1, 130, 8, 2, 64)])
def test_nope_equals_sdpa(B, T, Hq, Hkv, D):
    rng = np.random.default_rng(T + D)
    q, k, v = rng.standard_normal((B, T, Hq, D)), rng.standard_normal((B, T, Hkv, D)), rng.standard_normal(
        (B, T, Hkv, D))
    assert np.abs(oracle.softmax_attn(q, k, v) - _sdpa(q, k, v)).max() < 1e-12


def test_rope_2d_closed_form():
    x = np.zeros((1, 6, 1, 2))
    x[..., 0] = 1.0
    y = oracle.rope(x, theta=10000.0)
    for m in range(6):
        assert np.allclose(y[0, m, 0], [math.cos(m), math.sin(m)], atol=1e-14)


def test_rope_pair_norms_and_frequencies():
    rng = np.random.default_rng(1)
    D, theta = 16, 500.0
    x = rng.standard_normal((2, 9, 3, D))
    y = oracle.rope(x, theta=theta, pos0=4)
    nx = np.hypot(x[..., 0::2], x[..., 1::2])
    ny = np.hypot(y[..., 0::2], y[..., 1::2])
    assert np.abs(nx - ny).max() < 1e-12
    # unit vector on pair p, one position later: turned by theta^(-2p/D)
    for p in range(D // 2):
        e = np.zeros((1, 2, 1, D))
        e[..., 2 * p] = 1.0
        r = oracle.rope(e, theta=theta)
        ang = theta ** (-2.0 * p / D)
        assert np.allclose(r[0, 1, 0, 2 * p:2 * p + 2], [math.cos(ang), math.sin(ang)], atol=1e-13)
        assert np.allclose(np.delete(r[0, 1, 0], [2 * p, 2 * p + 1]), 0.0)


def test_rope_scores_depend_on_position_difference():
    rng = np.random.default_rng(2)
    D = 32
    qv, kv = rng.standard_normal(D), rng.standard_normal(D)
    seq = np.zeros((1, 40, 1, D))
    seq[0, :, 0] = qv
    rq = oracle.rope(seq)
    seq[0, :, 0] = kv
    rk = oracle.rope(seq)
    for i, j, s in [(5, 2, 7), (30, 30, 3), (10, 0, 29)]:
        a = rq[0, i, 0] @ rk[0, j, 0]
        b = rq[0, i + s, 0] @ rk[0, j + s, 0]
        assert abs(a - b) < 1e-10 * (1 + abs(a))
    # and a different difference gives a different score (the rotation is not trivial)
    assert abs(rq[0, 5, 0] @ rk[0, 2, 0] - rq[0, 5, 0] @ rk[0, 3, 0]) > 1e-6


def test_rope_attention_is_sdpa_on_rotated_inputs():
    rng = np.random.default_rng(3)
    B, T, Hq, Hkv, D = 2, 50, 4, 1, 16
    q, k, v = rng.standard_normal((B, T, Hq, D)), rng.standard_normal((B, T, Hkv, D)), rng.standard_normal(
        (B, T, Hkv, D))
    o = oracle.softmax_attn(q, k, v, rope_theta=10000.0)
    assert np.abs(o - _sdpa(oracle.rope(q), oracle.rope(k), v)).max() < 1e-12
    assert np.abs(o - oracle.softmax_attn(q, k, v)).max() > 1e-3  # the rotation matters


@pytest.mark.parametrize("theta", [0.0, 10000.0])
def test_softmax_decode_is_last_row(theta):
    rng = np.random.default_rng(4)
    B, T, Hq, Hkv, D = 2, 33, 4, 2, 16
    q, k, v = rng.standard_normal((B, T, Hq, D)), rng.standard_normal((B, T, Hkv, D)), rng.standard_normal(
        (B, T, Hkv, D))
    full = oracle.softmax_attn(q, k, v, rope_theta=theta)
    kr = oracle.rope(k, theta) if theta > 0 else k  # a RoPE cache holds rotated keys
    kc = np.concatenate([kr, rng.standard_normal((B, 7, Hkv, D))], axis=1)  # slots past cache_len unused
    vc = np.concatenate([v, rng.standard_normal((B, 7, Hkv, D))], axis=1)
    dec = oracle.softmax_decode(q[:, T - 1], kc, vc, T, rope_theta=theta)
    assert np.abs(dec - full[:, T - 1]).max() < 1e-13


def test_identical_keys_give_mean_of_values():
    rng = np.random.default_rng(5)
    T, D = 12, 8
    k = np.tile(rng.standard_normal(D), (1, T, 1, 1))
    q, v = rng.standard_normal((1, T, 1, D)), rng.standard_normal((1, T, 1, D))
    o = oracle.softmax_attn(q, k, v)
    for i in range(T):
        assert np.allclose(o[0, i, 0], v[0, :i + 1, 0].mean(axis=0), atol=1e-13)


def test_rotated_bf16_rounding_matches_torch():
    """oracle.rope(..., bf16=True) -- the definition of atma_rope's bf16 output -- is the exact
    rotation rounded once as torch rounds fp64 -> bf16, over 262144 values at large positions and
    magnitudes from 2^-20 to 2^20."""
    rng = np.random.default_rng(6)
    x = rng.standard_normal((2, 512, 4, 64)) * np.exp2(rng.integers(-20, 21, size=(2, 512, 4, 64)))
    for pos0 in (0, 77, 262000):
        y = oracle.rope(x, 10000.0, pos0=pos0)
        ref = torch.from_numpy(y).to(torch.float32).to(torch.bfloat16).double().numpy()
        assert np.array_equal(oracle.rope(x, 10000.0, pos0=pos0, bf16=True), ref)


def _bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(torch.float32).to(torch.bfloat16).double().numpy()


LAMBDA = 7.0


@pytest.mark.parametrize("B,T,Hq,Hkv,D,qscale,theta", [(1, 400, 2, 1, 64, 1.0, 10000.0), (2, 90, 4, 2, 16, 4.0, 500.0),
                                                        (1, 300, 1, 1, 128, 2.0, 10000.0)])
def test_rope_rounding_tolerance_covers_rounding(B, T, Hq, Hkv, D, qscale, theta):
    """Rounding every rotated q and k element to bf16 (what a bf16 attention kernel consumes) moves
    each output element by less than the tolerance; so do random perturbations of the rotated
    operands within the same relative size 2^-8 (bf16's unit roundoff).  The actual rounding reaches at least a fifth of
    the tolerance somewhere (it is not vacuous)."""
    rng = np.random.default_rng(T + D)
    q = rng.standard_normal((B, T, Hq, D)) * qscale
    k, v = rng.standard_normal((B, T, Hkv, D)), rng.standard_normal((B, T, Hkv, D))
    o, tol = oracle.softmax_attn(q, k, v, rope_theta=theta, tol_lambda=LAMBDA)
    assert np.all(tol >= 0)
    rq, rk = oracle.rope(q, theta), oracle.rope(k, theta)
    moved = np.abs(oracle.softmax_attn(_bf16(rq), _bf16(rk), v) - o)
    assert np.all(moved <= tol + 1e-15)
    assert np.max(moved[:, 1:] / tol[:, 1:]) > 0.2
    for _ in range(3):
        pq = rq * (1 + rng.uniform(-1, 1, rq.shape) / 256)
        pk = rk * (1 + rng.uniform(-1, 1, rk.shape) / 256)
        assert np.all(np.abs(oracle.softmax_attn(pq, pk, v) - o) <= tol + 1e-15)


def test_rope_rounding_tolerance_zero_and_linear():
    """A single visible key leaves nothing to move (the first row of a causal sequence equals its
    value row whatever the logits), so the tolerance is zero there; it is linear in lambda; and
    for a two-key row it is lambda u sqrt(sum_j w_j^2 (v_j - o)^2 sum_e (q_e k_je)^2 +
    sum_e (q_e sum_j w_j k_je (v_j - o))^2) / sqrt(D), checked against perturbing each rotated
    element alone by u and summing the squared first-order responses (finite differences)."""
    rng = np.random.default_rng(11)
    D, u = 8, 2.0 ** -8
    q, k, v = (rng.standard_normal((1, 2, 1, D)) for _ in range(3))
    o, tol = oracle.softmax_attn(q, k, v, tol_lambda=LAMBDA)
    _, tol2 = oracle.softmax_attn(q, k, v, tol_lambda=2 * LAMBDA)
    assert np.all(tol[0, 0] == 0.0)
    assert np.allclose(tol2, 2 * tol, rtol=1e-12)
    # finite-difference responses of row 1 to each element of q_1, k_0, k_1 scaled by (1 + u)
    resp = []
    for which, j in (("q", 1), ("k", 0), ("k", 1)):
        for e in range(D):
            qq, kk = q.copy(), k.copy()
            if which == "q":
                qq[0, j, 0, e] *= 1 + 1e-6
            else:
                kk[0, j, 0, e] *= 1 + 1e-6
            resp.append((oracle.softmax_attn(qq, kk, v)[0, 1, 0] - o[0, 1, 0]) / 1e-6 * u)
    resp = np.array(resp)
    # q_1 is shared by both logits: its responses are the A terms; the key terms are the B terms
    expect = LAMBDA * np.sqrt(np.sum(resp ** 2, axis=0))
    assert np.allclose(tol[0, 1, 0], expect, rtol=1e-4)
