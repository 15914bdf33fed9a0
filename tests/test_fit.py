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


def _wg(W_O, g, G, D):
    return np.concatenate([W_O[(g * G + i) * D:(g * G + i + 1) * D] for i in range(G)], axis=1)


def _latent_output(f, V, g, G, r, dm):
    """V.B.C for KV head g's query heads, from the fitted B and W_ofT."""
    B = f["B"][g].astype(np.float64)
    C = np.concatenate([f["W_ofT"][:, (g * G + i) * r:(g * G + i + 1) * r].T for i in range(G)], axis=1)
    return V @ B @ C.astype(np.float64)


def test_output_fit_is_exact_for_a_low_rank_output_map():
    """With each group's output map W_g of rank r, the reduced-rank fit
    reproduces every output exactly, on Values it never saw."""
    rng = np.random.default_rng(5)
    H, G, D, r, dm, n = 2, 2, 16, 3, 10, 300
    W_O = np.zeros((H * G * D, dm))
    for g in range(H):
        Wg = rng.standard_normal((D, r)) @ rng.standard_normal((r, G * dm))
        for i in range(G):
            W_O[(g * G + i) * D:(g * G + i + 1) * D] = Wg[:, i * dm:(i + 1) * dm]
    V = rng.standard_normal((n, H, D))
    K = rng.standard_normal((n, H, D))
    f = fit.fit_output_aware(K, V, W_O, H * G, r, 2)
    Vnew = rng.standard_normal((50, H, D))
    for g in range(H):
        np.testing.assert_allclose(_latent_output(f, Vnew[:, g], g, G, r, dm), Vnew[:, g] @ _wg(W_O, g, G, D),
                                   atol=1e-4, rtol=1e-4)


def test_output_fit_beats_the_value_basis_on_the_output():
    """Both fits produce rank-r maps V -> output; the reduced-rank one is the
    least-squares optimum, so its output error is never larger than that of
    the Value basis folded into W_O (B.B^T.W_g)."""
    rng = np.random.default_rng(6)
    H, G, D, r, dm, n = 1, 4, 24, 5, 12, 400
    W_O = rng.standard_normal((H * G * D, dm))
    V = rng.standard_normal((n, H, D)) * np.linspace(2, 0.5, D)
    K = rng.standard_normal((n, H, D))
    f_out = fit.fit_output_aware(K, V, W_O, H * G, r, 2)
    f_val = fit.fit_factors(K, V, r, 2)
    Y = V[:, 0] @ _wg(W_O, 0, G, D)
    B = f_val["B"][0].astype(np.float64)
    err_val = np.linalg.norm(V[:, 0] @ B @ B.T @ _wg(W_O, 0, G, D) - Y)
    err_out = np.linalg.norm(_latent_output(f_out, V[:, 0], 0, G, r, dm) - Y)
    assert err_out <= err_val * (1 + 1e-6)
    assert err_out < 0.95 * err_val  # strictly better on a generic map


def _joint_residual(O, W_O, B, WofT):
    n, Hq, D = O.shape
    G, r = Hq // B.shape[0], B.shape[2]
    Y = sum(O[:, h] @ W_O[h * D:(h + 1) * D] for h in range(Hq))
    Yh = sum(O[:, h] @ B[h // G] @ WofT[:, h * r:(h + 1) * r].T for h in range(Hq))
    return np.linalg.norm(Yh - Y)


def test_joint_projection_recovers_a_planted_map():
    """W_O[h] = B_g(h).M_h makes the layer output exactly Σ_h (o_h.B_g).M_h:
    the joint fit returns every M_h, which only the right head -> group map
    and orientation can do (the two groups' bases differ)."""
    rng = np.random.default_rng(8)
    H, G, D, r, dm, n = 2, 2, 8, 3, 5, 200
    B = rng.standard_normal((H, D, r))
    M = rng.standard_normal((H * G, r, dm))
    W_O = np.concatenate([B[h // G] @ M[h] for h in range(H * G)])
    O = rng.standard_normal((n, H * G, D))
    WofT = fit.fit_joint_projection(O, W_O, B)
    assert WofT.shape == (dm, H * G * r)
    for h in range(H * G):
        np.testing.assert_allclose(WofT[:, h * r:(h + 1) * r], M[h].T, atol=1e-4)
    assert _joint_residual(O, W_O, B, WofT.astype(np.float64)) < 1e-3


def test_joint_projection_beats_per_head_and_per_partition_fits():
    """On outputs correlated across heads, the joint least-squares fit leaves
    a smaller error on the summed output than folding B^T.W_O per head or
    fitting each partition (half the heads, as on another GPU) against its
    own part of the output; never larger, as the joint optimum."""
    rng = np.random.default_rng(9)
    H, G, D, r, dm, n = 4, 2, 12, 3, 16, 600
    Hq = H * G
    shared = rng.standard_normal((n, D))  # a component every head's output carries
    O = 0.7 * shared[:, None, :] + rng.standard_normal((n, Hq, D))
    W_O = rng.standard_normal((Hq * D, dm))
    B = np.stack([_orthonormal(rng, D, r) for _ in range(H)])
    joint = fit.fit_joint_projection(O, W_O, B).astype(np.float64)
    fold = np.concatenate([B[h // G].T @ W_O[h * D:(h + 1) * D] for h in range(Hq)]).T
    half = Hq // 2
    part = np.concatenate([fit.fit_joint_projection(O[:, p * half:(p + 1) * half],
                                                    W_O[p * half * D:(p + 1) * half * D],
                                                    B[p * H // 2:(p + 1) * H // 2]).astype(np.float64)
                           for p in range(2)], axis=1)
    e_joint, e_fold, e_part = (_joint_residual(O, W_O, B, x) for x in (joint, fold, part))
    assert e_joint <= e_part * (1 + 1e-9) and e_joint <= e_fold * (1 + 1e-9)
    assert e_joint < 0.97 * e_part and e_part < e_fold


def test_joint_projection_rejects_bad_shapes():
    with pytest.raises(ValueError):
        fit.fit_joint_projection(np.zeros((10, 3, 8)), np.zeros((24, 4)), np.zeros((2, 8, 2)))  # 3 % 2
    with pytest.raises(ValueError):
        fit.fit_joint_projection(np.zeros((10, 4, 8)), np.zeros((30, 4)), np.zeros((2, 8, 2)))
