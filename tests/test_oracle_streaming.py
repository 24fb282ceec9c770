"""Pins of the oracle's streaming fit (gram, fit_from_gram, project) against closed forms and
against the independent SVD route of fit_anchor."""
import numpy as np

import oracle


def _planted(rng, M, T, d, sig):
    """delta = P diag(sig) Q^T with orthonormal P [T, k], Q [d, k] (k = len(sig))."""
    out, Qs = [], []
    for _ in range(M):
        P, _ = np.linalg.qr(rng.standard_normal((T, len(sig))))
        Q, _ = np.linalg.qr(rng.standard_normal((d, len(sig))))
        out.append((P * sig) @ Q.T)
        Qs.append(Q)
    return np.stack(out), np.stack(Qs)


def test_gram_of_a_planted_delta_is_q_sigma2_qt():
    rng = np.random.default_rng(1)
    sig = np.array([5.0, 3.0, 2.0, 0.5])
    D, Q = _planted(rng, 3, 40, 16, sig)
    G = oracle.gram(D)
    for m in range(3):
        np.testing.assert_allclose(G[m], (Q[m] * sig**2) @ Q[m].T, atol=1e-12)
    # trace = squared Frobenius norm = sum of sigma^2
    np.testing.assert_allclose(np.trace(G, axis1=1, axis2=2), np.sum(sig**2), rtol=1e-13)


def test_gram_is_additive_over_appended_rows():
    rng = np.random.default_rng(2)
    D = rng.standard_normal((2, 70, 8))
    G = oracle.gram(D)
    G1 = oracle.gram(D[:, :25])
    G2 = oracle.gram(D[:, 25:])
    np.testing.assert_allclose(G1 + G2, G, atol=1e-12)
    # and it is symmetric positive semi-definite
    np.testing.assert_array_equal(G, np.swapaxes(G, 1, 2))
    assert np.linalg.eigvalsh(G).min() > -1e-12


def test_fit_from_gram_matches_the_svd_route():
    rng = np.random.default_rng(3)
    D = rng.standard_normal((4, 60, 12)) * np.linspace(3.0, 0.2, 12)
    a = oracle.fit_anchor(D, 5)
    b = oracle.fit_from_gram(oracle.gram(D), 5)
    np.testing.assert_allclose(b["eig"], a["eig"], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(b["W"], a["W"], atol=1e-9)
    np.testing.assert_array_equal(b["k_eff"], a["k_eff"])
    np.testing.assert_allclose(oracle.project(D, b["W"]), a["U"], atol=1e-9)


def test_fit_from_a_planted_gram_and_the_truncation_error():
    rng = np.random.default_rng(4)
    sig = np.array([4.0, 2.0, 1.0, 0.5, 0.25])
    D, Q = _planted(rng, 2, 50, 10, sig)
    out = oracle.fit_from_gram(oracle.gram(D), 3)
    lam = np.zeros(10)
    lam[:5] = sig**2
    np.testing.assert_allclose(out["eig"], np.tile(lam, (2, 1)), atol=1e-12)
    for m in range(2):
        # W spans the top-3 planted directions, with the canonical sign
        np.testing.assert_allclose(np.abs(out["W"][m] @ Q[m][:, :3]), np.eye(3), atol=1e-10)
        assert np.all(out["W"][m][np.arange(3), np.argmax(np.abs(out["W"][m]), axis=1)] > 0)
        # Eckart-Young: the truncation keeps exactly the tail energy out
        U = oracle.project(D[m:m + 1], out["W"][m:m + 1])[0]
        np.testing.assert_allclose(np.sum((D[m] - U @ out["W"][m]) ** 2), np.sum(sig[3:] ** 2),
                                   rtol=1e-10)
    # 90% of 21.3125: 16 + 4 = 20 >= 19.18 at k = 2
    np.testing.assert_array_equal(out["k_eff"], [2, 2])


def test_zero_gram_gives_rank_zero():
    out = oracle.fit_from_gram(np.zeros((1, 6, 6)), 2)
    assert out["k_eff"][0] == 0 and np.all(out["eig"] == 0)
