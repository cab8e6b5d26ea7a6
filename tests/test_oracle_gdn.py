"""Pins for the GDN/KDA oracle: the printed delta-rule example, the unit-key
identities of the gradient-step backup slide, special-case reductions, and an
independent second algorithm (the chunked WY form) for the same result."""
import json
import os

import numpy as np
import pytest

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rand(seed, B, T, H, dk, dv, kda):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, T, H, dk)).astype(np.float32)
    k = rng.standard_normal((B, T, H, dk)).astype(np.float32)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, dv)).astype(np.float32)
    ashape = (B, T, H, dk) if kda else (B, T, H)
    alpha = rng.uniform(0.9, 1.0, ashape).astype(np.float32)
    beta = (1 / (1 + np.exp(-rng.standard_normal((B, T, H))))).astype(np.float32)
    S0 = rng.standard_normal((B, H, dk, dv))
    return q, k, v, alpha, beta, S0


def test_delta_rule_example():
    with open(os.path.join(GOLD, "delta_rule_example.json")) as f:
        g = json.load(f)
    one = np.ones((1, 1, 1, 1), np.float32)
    S, o = oracle.gdn(one, one, np.full((1, 1, 1, 1), g["target"], np.float32),
                      np.ones((1, 1, 1), np.float32), np.full((1, 1, 1), g["beta"], np.float32),
                      S0=np.full((1, 1, 1, 1), g["prediction"]))
    assert o.item() == g["expected_new_prediction"]
    assert S.item() == g["expected_new_prediction"]


def test_unit_key_gradient_step_identities():
    # backup slide "the delta rule is a local gradient step": for |kappa| = 1,
    # W_new kappa = (1-beta) W_old kappa + beta v, and for any u,
    # (W_new - W_old) u = beta (v - W_old kappa)(kappa^T u).  Here S = W^T.
    rng = np.random.default_rng(0)
    dk, dv = 7, 5
    for trial in range(5):
        # an exactly unit-norm fp32 key: four entries of +-1/2 at random positions
        kap = np.zeros(dk, np.float32)
        kap[rng.choice(dk, 4, replace=False)] = rng.choice([-0.5, 0.5], 4)
        v = rng.standard_normal(dv).astype(np.float32)
        beta = np.float32(rng.uniform(0.05, 0.95))
        S0 = rng.standard_normal((1, 1, dk, dv))
        S, _ = oracle.gdn(kap.reshape(1, 1, 1, dk), kap.reshape(1, 1, 1, dk), v.reshape(1, 1, 1, dv),
                          np.ones((1, 1, 1), np.float32), np.full((1, 1, 1), beta, np.float32), S0=S0)
        Wold, Wnew = S0[0, 0].T, S[0, 0].T
        kd = kap.astype(np.float64)
        beta, v = np.float64(beta), v.astype(np.float64)
        np.testing.assert_allclose(Wnew @ kd, (1 - beta) * (Wold @ kd) + beta * v, atol=1e-12)
        u = rng.standard_normal(dk)
        np.testing.assert_allclose((Wnew - Wold) @ u,
                                   beta * (v - Wold @ kd) * (kd @ u), atol=1e-12)


def test_kda_with_uniform_channels_is_gdn():
    q, k, v, a, beta, S0 = _rand(1, 2, 11, 2, 6, 5, kda=False)
    a_ch = np.repeat(a[..., None], 6, axis=-1)
    S1, o1 = oracle.gdn(q, k, v, a, beta, S0, kda=False)
    S2, o2 = oracle.gdn(q, k, v, a_ch, beta, S0, kda=True)
    np.testing.assert_array_equal(S1, S2)
    np.testing.assert_array_equal(o1, o2)


def test_no_write_is_pure_decay():
    q, k, v, a, beta, S0 = _rand(2, 1, 6, 1, 4, 3, kda=True)
    S, o = oracle.gdn(q, k, v, a, np.zeros_like(beta), S0, kda=True)
    cum = np.cumprod(a[0, :, 0].astype(np.float64), axis=0)  # [T, dk]
    np.testing.assert_allclose(S[0, 0], cum[-1][:, None] * S0[0, 0], atol=1e-13)
    for t in range(6):
        np.testing.assert_allclose(o[0, t, 0], (cum[t][:, None] * S0[0, 0]).T @ q[0, t, 0], atol=1e-12)


def test_orthonormal_keys_store_exactly():
    # alpha = 1, beta = 1, keys are basis vectors: each write replaces the
    # association exactly, so reading at key e_j returns v_j
    dk, dv, T = 5, 3, 5
    rng = np.random.default_rng(4)
    k = np.eye(dk, dtype=np.float32)[:T].reshape(1, T, 1, dk)
    v = rng.standard_normal((1, T, 1, dv)).astype(np.float32)
    S, _ = oracle.gdn(k, k, v, np.ones((1, T, 1), np.float32), np.ones((1, T, 1), np.float32),
                      S0=rng.standard_normal((1, 1, dk, dv)))
    np.testing.assert_allclose(S[0, 0], v[0, :, 0].astype(np.float64), atol=1e-15)


def _chunked_wy(q, k, v, alpha, beta, S0, kda, C):
    """Chunked form of the same recurrence, written from its closed form:
    inside a chunk with cumulative log-decay lam_t,
      (I + A) U = diag(beta) (V - (K * e^lam) S0),  A[t,j] = beta_t k_t.(e^{lam_t-lam_j} k_j), j<t
      o_t = (q_t * e^{lam_t}) S0 + sum_{j<=t} (q_t.(e^{lam_t-lam_j} k_j)) u_j
      S_C = e^{lam_C} S0 + sum_j (e^{lam_C-lam_j} k_j) u_j^T
    """
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    q, k, v = (x.astype(np.float64) for x in (q, k, v))
    la = np.log(alpha.astype(np.float64))
    if not kda:
        la = np.repeat(la[..., None], dk, axis=-1)
    beta = beta.astype(np.float64)
    S_out = np.zeros((B, H, dk, dv))
    o = np.zeros((B, T, H, dv))
    for b in range(B):
        for h in range(H):
            S = S0[b, h].copy()
            for c0 in range(0, T, C):
                sl = slice(c0, min(T, c0 + C))
                K, Q, V, Bt = k[b, sl, h], q[b, sl, h], v[b, sl, h], beta[b, sl, h]
                lam = np.cumsum(la[b, sl, h], axis=0)  # [L, dk]
                L = K.shape[0]
                D = np.exp(lam[:, None, :] - lam[None, :, :])  # [t, j, dk]
                G = np.einsum("ti,tji,ji->tj", K, D, K)
                P = np.einsum("ti,tji,ji->tj", Q, D, K)
                A = np.tril(Bt[:, None] * G, -1)
                U = np.linalg.solve(np.eye(L) + A, Bt[:, None] * (V - (K * np.exp(lam)) @ S))
                o[b, sl, h] = (Q * np.exp(lam)) @ S + np.tril(P) @ U
                S = np.exp(lam[-1])[:, None] * S + (K * np.exp(lam[-1] - lam)).T @ U
            S_out[b, h] = S
    return S_out, o


@pytest.mark.parametrize("kda", [False, True])
def test_sequential_equals_chunked_form(kda):
    q, k, v, a, beta, S0 = _rand(9 + kda, 2, 37, 2, 8, 6, kda)
    S, o = oracle.gdn(q, k, v, a, beta, S0, kda=kda)
    S2, o2 = _chunked_wy(q, k, v, a, beta, S0, kda, C=16)
    np.testing.assert_allclose(S, S2, rtol=0, atol=1e-10)
    np.testing.assert_allclose(o, o2, rtol=0, atol=1e-10)


# ---------------- GDN2: key-side erase b, value-side write w ----------------

def test_gdn2_with_b_w_equal_beta_is_kda():
    # slide "GDN2 separates key-side erase and value-side write": b = w = beta 1 recovers KDA
    q, k, v, a, beta, S0 = _rand(21, 2, 19, 2, 8, 6, True)
    bb = np.repeat(beta[..., None], 8, axis=-1)
    ww = np.repeat(beta[..., None], 6, axis=-1)
    S2, o2 = oracle.gdn2(q, k, v, a, bb, ww, S0)
    S1, o1 = oracle.gdn(q, k, v, a, beta, S0, kda=True)
    np.testing.assert_allclose(S2, S1, rtol=0, atol=1e-12)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-12)


def test_gdn2_first_token_closed_form():
    # from an empty state the residual is the write target: S = kappa (w . v)^T, o = (kappa.q)(w . v)
    rng = np.random.default_rng(22)
    dk, dv = 6, 5
    q = rng.standard_normal((1, 1, 1, dk)).astype(np.float32)
    k = rng.standard_normal((1, 1, 1, dk)).astype(np.float32)
    v = rng.standard_normal((1, 1, 1, dv)).astype(np.float32)
    a = rng.uniform(0.5, 1, (1, 1, 1, dk)).astype(np.float32)
    b = rng.uniform(0, 1, (1, 1, 1, dk)).astype(np.float32)
    w = rng.uniform(0, 1, (1, 1, 1, dv)).astype(np.float32)
    S, o = oracle.gdn2(q, k, v, a, b, w)
    z = w[0, 0, 0].astype(np.float64) * v[0, 0, 0]
    kk = k[0, 0, 0].astype(np.float64)
    np.testing.assert_allclose(S[0, 0], np.outer(kk, z), rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(o[0, 0, 0], (kk @ q[0, 0, 0].astype(np.float64)) * z, rtol=1e-13)


def test_gdn2_erase_and_write_roles():
    # one stored association S0 = e_j u0^T, alpha = 1, same unit key e_j:
    # b = 1 erases it before the write (S = e_j (w.v)^T), b = 0 keeps it (S = e_j (u0 + w.v)^T);
    # w = 0 with b = 1 erases the key's association entirely (S^T e_j = 0)
    dk, dv, j = 4, 3, 2
    rng = np.random.default_rng(23)
    u0 = rng.standard_normal(dv)
    S0 = np.zeros((1, 1, dk, dv))
    S0[0, 0, j] = u0
    e = np.zeros((1, 1, 1, dk), np.float32)
    e[..., j] = 1
    v = rng.standard_normal((1, 1, 1, dv)).astype(np.float32)
    w = rng.uniform(0.2, 1, (1, 1, 1, dv)).astype(np.float32)
    one = np.ones((1, 1, 1, dk), np.float32)
    z = (w * v)[0, 0, 0].astype(np.float64)
    S, _ = oracle.gdn2(e, e, v, one, one, w, S0)
    np.testing.assert_allclose(S[0, 0, j], z, atol=1e-15)
    S, _ = oracle.gdn2(e, e, v, one, 0 * one, w, S0)
    np.testing.assert_allclose(S[0, 0, j], u0 + z, atol=1e-15)
    S, _ = oracle.gdn2(e, e, v, one, one, 0 * w, S0)
    np.testing.assert_allclose(S[0, 0, j], 0.0, atol=1e-15)


def _chunked_gdn2(q, k, v, alpha, b, w, S0, C):
    """Chunked form written from the GDN2 recurrence: with cumulative log-decay lam,
      (I + A) U = W.V - ((B.K) * e^lam) S0,  A[t,j] = (b_t.k_t).(e^{lam_t-lam_j} k_j), j<t
      o_t = (q_t * e^{lam_t}) S0 + sum_{j<=t} (q_t.(e^{lam_t-lam_j} k_j)) u_j
      S_C = e^{lam_C} S0 + sum_j (e^{lam_C-lam_j} k_j) u_j^T
    """
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    q, k, v, b, w = (x.astype(np.float64) for x in (q, k, v, b, w))
    la = np.log(alpha.astype(np.float64))
    S_out = np.zeros((B, H, dk, dv))
    o = np.zeros((B, T, H, dv))
    for bi in range(B):
        for h in range(H):
            S = S0[bi, h].copy()
            for c0 in range(0, T, C):
                sl = slice(c0, min(T, c0 + C))
                K, Q, V = k[bi, sl, h], q[bi, sl, h], v[bi, sl, h]
                E, Wv = b[bi, sl, h] * K, w[bi, sl, h] * V
                lam = np.cumsum(la[bi, sl, h], axis=0)
                L = K.shape[0]
                D = np.exp(lam[:, None, :] - lam[None, :, :])
                A = np.tril(np.einsum("ti,tji,ji->tj", E, D, K), -1)
                P = np.einsum("ti,tji,ji->tj", Q, D, K)
                U = np.linalg.solve(np.eye(L) + A, Wv - (E * np.exp(lam)) @ S)
                o[bi, sl, h] = (Q * np.exp(lam)) @ S + np.tril(P) @ U
                S = np.exp(lam[-1])[:, None] * S + (K * np.exp(lam[-1] - lam)).T @ U
            S_out[bi, h] = S
    return S_out, o


def test_gdn2_sequential_equals_chunked_form():
    q, k, v, a, _, S0 = _rand(24, 2, 41, 2, 8, 6, True)
    rng = np.random.default_rng(25)
    b = rng.uniform(0, 1, (2, 41, 2, 8)).astype(np.float32)
    w = rng.uniform(0, 1, (2, 41, 2, 6)).astype(np.float32)
    S, o = oracle.gdn2(q, k, v, a, b, w, S0)
    S2, o2 = _chunked_gdn2(q, k, v, a, b, w, S0, C=16)
    np.testing.assert_allclose(S, S2, rtol=0, atol=1e-10)
    np.testing.assert_allclose(o, o2, rtol=0, atol=1e-10)
