"""Pins of the oracle's Canon prologue (depthwise causal convolution over tokens, optional
residual, optional unit L2 norm per head), against what a library routine and the definition
fix: numpy's full convolution per channel, the impulse response, causality, the identity
kernel, continuation through the carried state, unit norms and scale invariance."""
import numpy as np
import pytest

import oracle


def test_equals_numpy_convolve_per_channel():
    rng = np.random.default_rng(0)
    B, T, C, K = 2, 37, 12, 4
    x, w = rng.standard_normal((B, T, C)), rng.standard_normal((K, C))
    y = oracle.canon(x, w)
    for b in range(B):
        for c in range(C):
            assert np.allclose(y[b, :, c], np.convolve(x[b, :, c], w[:, c])[:T], atol=1e-13)


def test_impulse_response_and_causality():
    rng = np.random.default_rng(1)
    T, C, K, t0 = 20, 5, 4, 7
    w = rng.standard_normal((K, C))
    x = np.zeros((1, T, C))
    x[0, t0] = 1.0
    y = oracle.canon(x, w)
    for t in range(T):
        expect = w[t - t0] if 0 <= t - t0 < K else np.zeros(C)
        assert np.allclose(y[0, t], expect, atol=1e-14)
    x2 = rng.standard_normal((1, T, C))
    x3 = x2.copy()
    x3[0, 12:] += 5.0
    assert np.allclose(oracle.canon(x2, w)[0, :12], oracle.canon(x3, w)[0, :12], atol=1e-14)


def test_identity_kernel_and_residual():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((2, 9, 6))
    w = np.ones((1, 6))
    assert np.allclose(oracle.canon(x, w), x, atol=1e-15)
    assert np.allclose(oracle.canon(x, w, residual=True), 2 * x, atol=1e-15)


@pytest.mark.parametrize("split", [1, 2, 5, 20])
def test_state_continues_the_sequence(split):
    rng = np.random.default_rng(3)
    B, T, C, K = 2, 25, 8, 4
    x, w = rng.standard_normal((B, T, C)), rng.standard_normal((K, C))
    full = oracle.canon(x, w, residual=True)
    head = oracle.canon(x[:, :split], w, residual=True)
    pad = np.concatenate([np.zeros((B, K - 1, C)), x[:, :split]], axis=1)
    state = pad[:, -(K - 1):]
    tail = oracle.canon(x[:, split:], w, state=state, residual=True)
    assert np.allclose(np.concatenate([head, tail], axis=1), full, atol=1e-13)


def test_head_norm_unit_and_scale_invariant():
    rng = np.random.default_rng(4)
    B, T, H, D, K = 1, 11, 3, 8, 3
    x, w = rng.standard_normal((B, T, H * D)), rng.standard_normal((K, H * D))
    y = oracle.canon(x, w, heads=H).reshape(B, T, H, D)
    assert np.allclose(np.linalg.norm(y, axis=-1), 1.0, atol=1e-13)
    y2 = oracle.canon(3.5 * x, w, heads=H).reshape(B, T, H, D)
    assert np.allclose(y, y2, atol=1e-13)
    raw = oracle.canon(x, w).reshape(B, T, H, D)
    assert np.allclose(y, raw / np.linalg.norm(raw, axis=-1, keepdims=True), atol=1e-13)
