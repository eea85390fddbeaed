"""Pins for the fp64 gated-delta-memory oracle (CPU only).

Each test checks the oracle against something other than itself: a closed form
that follows from the recurrence of the ATMA paper (Section 3.3 equation), an
invariant stated in Appendix A.2, or an exact identity (chunked == sequential,
resume == one pass).  Mistakes such as a flipped sign in (I - beta k k^T), a
transposed state, reading S_{t-1} instead of S_t for the output, applying the decay
to only one term, or a wrong time index each break at least one of these tests.
"""
import numpy as np
import pytest

import oracle


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _inputs(rng, B, T, H, Dk, Dv, alpha_range=(0.6, 0.999)):
    q = _unit(rng.standard_normal((B, T, H, Dk)))
    k = _unit(rng.standard_normal((B, T, H, Dk)))
    v = rng.standard_normal((B, T, H, Dv))
    alpha = rng.uniform(*alpha_range, size=(B, T, H))
    beta = rng.uniform(0.0, 1.0, size=(B, T, H))
    return q, k, v, alpha, beta


def test_beta_zero_is_pure_decay(rng):
    """beta = 0: S_t = (prod_{s<=t} alpha_s) S_0 and o_t = (prod_{s<=t} alpha_s) S_0 q_t."""
    B, T, H, Dk, Dv = 2, 37, 3, 8, 5
    q, k, v, alpha, _ = _inputs(rng, B, T, H, Dk, Dv)
    beta = np.zeros((B, T, H))
    S0 = rng.standard_normal((B, H, Dv, Dk))
    o, ST = oracle.gdn_sequential(q, k, v, alpha, beta, init_state=S0)
    decay = np.cumprod(alpha, axis=1)  # [B,T,H]
    exp_o = decay[..., None] * np.einsum("bhij,bthj->bthi", S0, q)
    exp_S = decay[:, -1][..., None, None] * S0
    np.testing.assert_allclose(o, exp_o, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(ST, exp_S, rtol=1e-12, atol=1e-13)


def test_orthonormal_keys_recall_exactly(rng):
    """alpha = beta = 1 with orthonormal keys: (I - k k^T) is a projector, so after writing
    (k_s, v_s) the state maps every stored key to its value, whatever S_0 was."""
    Dk, Dv, m = 16, 7, 16
    basis, _ = np.linalg.qr(rng.standard_normal((Dk, Dk)))
    keys = basis.T[:m]  # rows orthonormal
    vals = rng.standard_normal((m, Dv))
    q = np.repeat(keys[None, :, None, :], 1, axis=0)  # query each step with the key just written
    k = q.copy()
    v = vals[None, :, None, :]
    ones = np.ones((1, m, 1))
    S0 = rng.standard_normal((1, 1, Dv, Dk))
    o, ST = oracle.gdn_sequential(q, k, v, ones, ones, init_state=S0)
    np.testing.assert_allclose(o[0, :, 0], vals, atol=1e-12)
    np.testing.assert_allclose(ST[0, 0] @ keys.T, vals.T, atol=1e-12)


def test_repeated_key_returns_latest_value(rng):
    """alpha = beta = 1: writing the same key twice overwrites (needle update)."""
    Dk, Dv = 8, 4
    basis, _ = np.linalg.qr(rng.standard_normal((Dk, Dk)))
    seq_keys = [basis[:, 0], basis[:, 1], basis[:, 0], basis[:, 2]]
    vals = rng.standard_normal((4, Dv))
    k = np.stack(seq_keys)[None, :, None, :]
    q = np.repeat(basis[:, 0][None, None, None, :], 4, axis=1)
    v = vals[None, :, None, :]
    ones = np.ones((1, 4, 1))
    o, ST = oracle.gdn_sequential(q, k, v, ones, ones)
    np.testing.assert_allclose(o[0, 0, 0], vals[0], atol=1e-12)
    np.testing.assert_allclose(o[0, 1, 0], vals[0], atol=1e-12)
    np.testing.assert_allclose(o[0, 2, 0], vals[2], atol=1e-12)
    np.testing.assert_allclose(ST[0, 0] @ basis[:, 0], vals[2], atol=1e-12)
    np.testing.assert_allclose(ST[0, 0] @ basis[:, 1], vals[1], atol=1e-12)


def test_single_token_closed_form(rng):
    """T = 1: o = alpha S_0 (q - beta (k.q) k) + beta (k.q) v."""
    B, H, Dk, Dv = 3, 2, 6, 9
    q, k, v, alpha, beta = _inputs(rng, B, 1, H, Dk, Dv)
    S0 = rng.standard_normal((B, H, Dv, Dk))
    o, _ = oracle.gdn_sequential(q, k, v, alpha, beta, init_state=S0)
    for b in range(B):
        for h in range(H):
            qq, kk, vv = q[b, 0, h], k[b, 0, h], v[b, 0, h]
            a, be = alpha[b, 0, h], beta[b, 0, h]
            kq = kk @ qq
            want = a * S0[b, h] @ (qq - be * kq * kk) + be * kq * vv
            np.testing.assert_allclose(o[b, 0, h], want, rtol=1e-12, atol=1e-13)


def test_two_token_closed_form(rng):
    """T = 2 from a zero state:
    o_1 = beta_1 (k_1.q_1) v_1,
    o_2 = alpha_2 beta_1 (k_1.q_2 - beta_2 (k_1.k_2)(k_2.q_2)) v_1 + beta_2 (k_2.q_2) v_2."""
    Dk, Dv = 5, 3
    q, k, v, alpha, beta = _inputs(rng, 1, 2, 1, Dk, Dv)
    o, _ = oracle.gdn_sequential(q, k, v, alpha, beta)
    q1, q2 = q[0, 0, 0], q[0, 1, 0]
    k1, k2 = k[0, 0, 0], k[0, 1, 0]
    v1, v2 = v[0, 0, 0], v[0, 1, 0]
    a2 = alpha[0, 1, 0]
    b1, b2 = beta[0, 0, 0], beta[0, 1, 0]
    np.testing.assert_allclose(o[0, 0, 0], b1 * (k1 @ q1) * v1, rtol=1e-12)
    want2 = a2 * b1 * (k1 @ q2 - b2 * (k1 @ k2) * (k2 @ q2)) * v1 + b2 * (k2 @ q2) * v2
    np.testing.assert_allclose(o[0, 1, 0], want2, rtol=1e-12)


@pytest.mark.parametrize("chunk", [1, 7, 16, 64, 200])
def test_chunked_equals_sequential(rng, chunk):
    """The chunked rewrite (UT transform) reproduces the sequential recurrence, including a
    ragged last chunk and a non-zero initial state."""
    B, T, H, Dk, Dv = 2, 200, 2, 16, 24
    q, k, v, alpha, beta = _inputs(rng, B, T, H, Dk, Dv, alpha_range=(0.3, 1.0))
    S0 = rng.standard_normal((B, H, Dv, Dk))
    o1, S1 = oracle.gdn_sequential(q, k, v, alpha, beta, init_state=S0)
    o2, S2 = oracle.gdn_chunked(q, k, v, alpha, beta, init_state=S0, chunk=chunk)
    scale = np.sqrt(np.mean(o1 ** 2))
    assert np.max(np.abs(o1 - o2)) <= 1e-12 * scale
    assert np.max(np.abs(S1 - S2)) <= 1e-12 * np.sqrt(np.mean(S1 ** 2))


def test_state_norm_bound(rng):
    """Appendix A.2: ||S_t||_F <= abar^t ||S_0||_F + V / (1 - abar) for unit q, k,
    ||v|| <= V, 0 <= beta <= 1, 0 <= alpha <= abar < 1."""
    B, T, H, Dk, Dv = 1, 300, 2, 8, 8
    q, k, v, alpha, beta = _inputs(rng, B, T, H, Dk, Dv, alpha_range=(0.5, 0.97))
    beta[..., ::3] = 1.0
    S0 = 5.0 * rng.standard_normal((B, H, Dv, Dk))
    _, _, states = oracle.gdn_sequential(q, k, v, alpha, beta, init_state=S0, want_states=True)
    abar = alpha.max()
    V = np.linalg.norm(v, axis=-1).max()
    n0 = np.linalg.norm(S0.reshape(B, H, -1), axis=-1)  # [B,H]
    norms = np.linalg.norm(states.reshape(B, T, H, -1), axis=-1)  # [B,T,H]
    t = np.arange(1, T + 1)[None, :, None]
    bound = abar ** t * n0[:, None, :] + V / (1 - abar)
    assert np.all(norms <= bound * (1 + 1e-12))


def test_resume_and_decode_steps(rng):
    """Prefill(T1) then prefill(T2, init=final) equals prefill(T1+T2); so does a run of
    single-token steps."""
    B, T, H, D = 2, 23, 2, 6
    q, k, v, alpha, beta = _inputs(rng, B, T, H, D, D)
    S0 = rng.standard_normal((B, H, D, D))
    o, ST = oracle.gdn_sequential(q, k, v, alpha, beta, init_state=S0)
    T1 = 9
    oa, Sa = oracle.gdn_chunked(q[:, :T1], k[:, :T1], v[:, :T1], alpha[:, :T1], beta[:, :T1], S0, chunk=4)
    ob, Sb = oracle.gdn_chunked(q[:, T1:], k[:, T1:], v[:, T1:], alpha[:, T1:], beta[:, T1:], Sa, chunk=4)
    np.testing.assert_allclose(np.concatenate([oa, ob], axis=1), o, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(Sb, ST, rtol=1e-11, atol=1e-12)
    S = S0
    for t in range(T):
        ot, S = oracle.gdn_decode_step(q[:, t], k[:, t], v[:, t], alpha[:, t], beta[:, t], S)
        np.testing.assert_allclose(ot, o[:, t], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(S, ST, rtol=1e-11, atol=1e-12)


def test_heads_and_batches_are_independent(rng):
    """Each (batch, head) runs its own recurrence: permuting heads permutes outputs."""
    B, T, H, D = 2, 11, 3, 4
    q, k, v, alpha, beta = _inputs(rng, B, T, H, D, D)
    o, S = oracle.gdn_sequential(q, k, v, alpha, beta)
    perm = [2, 0, 1]
    o2, S2 = oracle.gdn_sequential(q[:, :, perm], k[:, :, perm], v[:, :, perm], alpha[:, :, perm],
                                   beta[:, :, perm])
    np.testing.assert_allclose(o2, o[:, :, perm], rtol=0, atol=0)
    np.testing.assert_allclose(S2, S[:, perm], rtol=0, atol=0)
