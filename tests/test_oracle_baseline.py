"""Pins of the oracle's NoPE / RoPE control cores (the matched baselines of the ATMA paper,
Section 3.1), checked against what mathematics and a library routine fix:

* NoPE equals torch's scaled-dot-product attention (causal, fp64) with kv heads repeated;
* RoPE rotates each adjacent pair: a D=2 unit vector at position m becomes (cos m, sin m);
  pair norms are preserved; pair p turns by theta^(-2p/D) per position (the textbook
  frequencies); scores depend only on the position difference (shift invariance);
* the decode row equals the last row of the causal forward, with and without RoPE;
* identical keys give the plain mean of the values.
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
    kc = np.concatenate([k, rng.standard_normal((B, 7, Hkv, D))], axis=1)  # slots past cache_len unused
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
    """The bf16 rounding of the rotation equals torch's fp64 -> bf16 conversion, and the core
    with rounded rotations is the NoPE core on those rounded values."""
    rng = np.random.default_rng(6)
    x = rng.standard_normal((2, 40, 3, 16)) * 3.0
    ref = torch.from_numpy(oracle.rope(x, 10000.0, pos0=77)).to(torch.bfloat16).double().numpy()
    assert np.array_equal(oracle.rope(x, 10000.0, pos0=77, bf16=True), ref)
    q, k, v = x[:, :, :2], x[:, :, 2:], rng.standard_normal((2, 40, 1, 16))
    o = oracle.softmax_attn(q, k, v, rope_theta=10000.0, rotated_bf16=True)
    o2 = oracle.softmax_attn(oracle.rope(q, bf16=True), oracle.rope(k, bf16=True), v)
    assert np.abs(o - o2).max() < 1e-13
