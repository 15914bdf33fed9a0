"""Offline factor fitting and the routing-recall measure (host numpy),
pinned by constructions whose answer is known exactly."""
import numpy as np
import pytest

from routed_decode_attention_amd import fit


def _orthonormal(rng, d, k):
    q, _ = np.linalg.qr(rng.standard_normal((d, k)))
    return q


def _projector(M):
    return M @ M.T


def test_value_basis_spans_a_planted_low_rank_subspace():
    rng = np.random.default_rng(1)
    n, D, r = 400, 32, 6
    M = _orthonormal(rng, D, r)
    V = (rng.standard_normal((n, r)) * np.linspace(3, 1, r)) @ M.T
    K = rng.standard_normal((n, D))
    f = fit.fit_factors(K[:, None], V[:, None], r, 2)
    B = f["B"][0].astype(np.float64)
    np.testing.assert_allclose(B.T @ B, np.eye(r), atol=1e-6)
    np.testing.assert_allclose(_projector(B), _projector(M), atol=1e-6)


def test_predictor_and_residual_recover_a_planted_key_model():
    """K = Z.P_true + S.R^T with S orthogonal to the latents: the least-squares
    predictor is P_true, and the residual code spans R exactly."""
    rng = np.random.default_rng(2)
    n, D, r, rk = 500, 24, 5, 3
    V = rng.standard_normal((n, D)) * np.concatenate([np.full(r, 4.0), np.ones(D - r)])
    f0 = fit.fit_factors(np.zeros((n, 1, D)), V[:, None], r, 1)
    Z = V @ f0["B"][0].astype(np.float64)
    P_true = rng.standard_normal((r, D))
    S = rng.standard_normal((n, rk))
    S -= Z @ np.linalg.lstsq(Z, S, rcond=None)[0]  # no part of S lies in the latents' span
    R = _orthonormal(rng, D, rk)
    K = Z @ P_true + S @ R.T
    f = fit.fit_factors(K[:, None], V[:, None], r, rk)
    np.testing.assert_allclose(f["P"][0], P_true, atol=1e-4)
    Re, Rd = f["R_enc"][0].astype(np.float64), f["R_dec"][0].astype(np.float64)
    np.testing.assert_allclose(_projector(Re), _projector(R), atol=1e-5)
    np.testing.assert_allclose(Rd, Re.T)
    E = K - Z @ f["P"][0].astype(np.float64)
    np.testing.assert_allclose(E @ Re @ Rd, E, atol=1e-4)


def test_fit_rejects_bad_ranks():
    with pytest.raises(ValueError):
        fit.fit_factors(np.zeros((4, 1, 8)), np.zeros((4, 1, 8)), 9, 1)
    with pytest.raises(ValueError):
        fit.fit_factors(np.zeros((4, 1, 8)), np.zeros((5, 1, 8)), 2, 1)


def test_page_mass_against_brute_force():
    rng = np.random.default_rng(3)
    n, Hk, G, D, ps = 37, 2, 2, 8, 8
    K = rng.standard_normal((n, Hk, D))
    q = rng.standard_normal((Hk * G, D))
    m = fit.page_mass(K, q, n, ps, G, scale=0.7)
    assert m.shape == (Hk * G, 5)
    for h in range(Hk * G):
        w = [np.exp(0.7 * sum(K[t, h // G, i] * q[h, i] for i in range(D))) for t in range(n)]
        tot = sum(w)
        for j in range(5):
            assert abs(m[h, j] - sum(w[t] for t in range(j * ps, min(n, (j + 1) * ps))) / tot) < 1e-12


def test_recall_bounds():
    rng = np.random.default_rng(4)
    m = rng.random((4, 10))
    m /= m.sum(axis=1, keepdims=True)
    assert fit.recall(m, range(10)) == pytest.approx(1.0)
    assert fit.recall(m, [-1, -1]) == 0.0
    # one page carrying every head's mass
    hot = np.zeros((3, 6))
    hot[:, 4] = 1.0
    assert fit.recall(hot, [4, -1]) == 1.0 and fit.recall(hot, [0, 1, 2, 3, 5]) == 0.0
    for k in range(1, 10):
        assert fit.best_recall(m, k) >= fit.recall(m, rng.choice(10, k, replace=False)) - 1e-12
