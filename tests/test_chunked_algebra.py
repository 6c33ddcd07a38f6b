"""The chunked (WY) form the GPU's GDN kernel evaluates equals the per-token recurrence.

This is a float64 NumPy model of the kernel's algebra (not of its code), checked
against the oracle's recurrence.  Derivation, for one chunk of n rows with start
state S0 [dv, dk], g_t = sum_{s<=t} log alpha_s and Gamma_ts = exp(g_t - g_s):

    u_t = eta_t (v_t - alpha_t S_{t-1} k_t)          so that S_t = alpha_t S_{t-1} + u_t k_t^T
    (I + A) U = diag(eta) V - diag(eta e^g) K S0^T,  A_ts = eta_t Gamma_ts k_t.k_s  (s < t)
    O = diag(e^g) Q S0^T + (tril(Gamma) * Q K^T) U
    S_n = e^{g_n} S0 + U^T diag(e^{g_n - g}) K

(the same kind of chunk algebra as the Gram / triangular-solve / forward
substitution steps of the rollback-free GDN verification in "기술 요약: 마진으로부터의
트리 (DFlash-TfM)", 방법론 §3).
"""
import numpy as np
import pytest

from oracle.gdn import gated_delta_rule


def chunked(q, k, v, alpha, eta, S0, C):
    L, dk = q.shape
    S = S0.copy()
    o = np.zeros((L, v.shape[1]))
    for c0 in range(0, L, C):
        sl = slice(c0, min(L, c0 + C))
        Q, K, V, a, e = q[sl], k[sl], v[sl], alpha[sl], eta[sl]
        n = Q.shape[0]
        g = np.cumsum(np.log(a))
        Gam = np.exp(g[:, None] - g[None, :])
        A = np.tril(e[:, None] * Gam * (K @ K.T), -1)
        Tinv = np.linalg.inv(np.eye(n) + A)
        Wm = Tinv @ ((e * np.exp(g))[:, None] * K)
        Ut = Tinv @ (e[:, None] * V)
        U = Ut - Wm @ S.T
        o[sl] = np.exp(g)[:, None] * (Q @ S.T) + (np.tril(Gam) * (Q @ K.T)) @ U
        S = np.exp(g[-1]) * S + U.T @ (np.exp(g[-1] - g)[:, None] * K)
    return o, S


@pytest.mark.parametrize("C", [1, 7, 16, 64])
def test_chunked_form_matches_recurrence(C):
    rng = np.random.default_rng(C)
    L, dk, dv = 150, 16, 12
    q = rng.standard_normal((L, dk))
    k = rng.standard_normal((L, dk))
    q /= np.linalg.norm(q, axis=1, keepdims=True)
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = rng.standard_normal((L, dv))
    alpha = 1 / (1 + np.exp(-(2 + 0.5 * rng.standard_normal(L))))
    eta = 1 / (1 + np.exp(-rng.standard_normal(L)))
    S0 = rng.standard_normal((dv, dk)) * 0.3
    o_ref, S_ref = gated_delta_rule(q[:, None], k[:, None], v[:, None], alpha[:, None], eta[:, None], S0[None])
    o, S = chunked(q, k, v, alpha, eta, S0, C)
    np.testing.assert_allclose(o, o_ref[:, 0], atol=1e-12)
    np.testing.assert_allclose(S, S_ref[0], atol=1e-12)
