"""Pins of the oracle's anchor fit: hand-worked SVDs, planted spectra, Eckart-Young,
brute force over directions, an independent power iteration and the effective-rank
closed forms."""
import json
import math
import os

import numpy as np
import pytest

import oracle
from conftest import GOLDEN


def _ev(x):
    if isinstance(x, str):
        return float(eval(x, {"sqrt": math.sqrt}))
    return float(x)


@pytest.mark.parametrize("case", json.load(open(os.path.join(GOLDEN, "fit_hand.json")))["cases"])
def test_fit_hand_cases(case):
    delta = np.array(case["delta"], dtype=np.float64)
    r = case["r"]
    out = oracle.fit_anchor(delta[None], r, 0.9)
    np.testing.assert_allclose(out["eig"][0], case["eig"], rtol=1e-14, atol=1e-13)
    for energy, k in case["k_eff"].items():
        assert int(oracle.effective_rank(out["eig"][0], float(energy))) == k
        assert int(oracle.fit_anchor(delta[None], r, float(energy))["k_eff"][0]) == k
    if case["W"] is not None:
        W = np.array([[_ev(v) for v in row] for row in case["W"]])
        np.testing.assert_allclose(out["W"][0], W, rtol=1e-14, atol=1e-14)
    U = np.array([[_ev(v) for v in row] for row in case["U"]])
    np.testing.assert_allclose(out["U"][0], U, rtol=1e-14, atol=1e-14)
    nd = np.linalg.norm(delta)
    err = np.linalg.norm(delta - out["U"][0] @ out["W"][0]) / (nd if nd > 0 else 1.0)
    assert err == pytest.approx(_ev(case["trunc_err"]), abs=1e-14)


def _planted(rng, T, d, sig):
    """delta = P diag(sig) Q^T with orthonormal P (T x k), Q (d x k): spectrum known exactly."""
    k = len(sig)
    P, _ = np.linalg.qr(rng.standard_normal((T, k)))
    Q, _ = np.linalg.qr(rng.standard_normal((d, k)))
    return P, Q, (P * sig) @ Q.T


def test_exact_rank_r_delta_is_recovered():
    rng = np.random.default_rng(0)
    T, d, r = 64, 16, 5
    sig = 7.0 * 0.8 ** np.arange(r)
    P, Q, delta = _planted(rng, T, d, sig)
    out = oracle.fit_anchor(delta[None], r)
    np.testing.assert_allclose(out["eig"][0, :r], sig ** 2, rtol=1e-12)
    np.testing.assert_allclose(out["eig"][0, r:], 0.0, atol=1e-24 + 1e-12 * sig[0] ** 2)
    rec = out["U"][0] @ out["W"][0]
    assert np.linalg.norm(rec - delta) / np.linalg.norm(delta) < 1e-12
    # W spans the planted right space, rows orthonormal, each row's largest entry positive
    np.testing.assert_allclose(out["W"][0] @ out["W"][0].T, np.eye(r), atol=1e-13)
    np.testing.assert_allclose(np.abs(out["W"][0] @ Q), np.eye(r), atol=1e-10)
    for row in out["W"][0]:
        assert row[np.argmax(np.abs(row))] > 0
    # U carries the singular values: ||U_i|| = sigma_i
    np.testing.assert_allclose(np.linalg.norm(out["U"][0], axis=0), sig, rtol=1e-12)


@pytest.mark.parametrize("r", [1, 3, 8, 15])
def test_eckart_young_against_planted_spectrum(r):
    rng = np.random.default_rng(r)
    T, d = 40, 16
    sig = np.sort(rng.uniform(0.1, 5.0, d))[::-1]
    _, _, delta = _planted(rng, T, d, sig)
    out = oracle.fit_anchor(delta[None], r)
    err = np.linalg.norm(delta - out["U"][0] @ out["W"][0]) / np.linalg.norm(delta)
    want = math.sqrt(float(np.sum(sig[r:] ** 2) / np.sum(sig ** 2)))
    assert err == pytest.approx(want, rel=1e-10, abs=1e-14)


def test_truncation_beats_random_rank_r_candidates():
    rng = np.random.default_rng(21)
    T, d, r = 12, 6, 2
    delta = rng.standard_normal((T, d))
    out = oracle.fit_anchor(delta[None], r)
    best = np.linalg.norm(delta - out["U"][0] @ out["W"][0])
    for _ in range(3000):
        Q, _ = np.linalg.qr(rng.standard_normal((d, r)))
        cand = delta @ Q @ Q.T  # best approximation within that row space
        assert np.linalg.norm(delta - cand) >= best - 1e-12


def test_brute_force_top_direction_2d():
    # d = 2: scan unit vectors v(theta); the top right singular vector maximises ||delta v||.
    rng = np.random.default_rng(5)
    delta = rng.standard_normal((7, 2))
    th = np.linspace(0.0, np.pi, 200001)
    vs = np.stack([np.cos(th), np.sin(th)])
    norms = np.linalg.norm(delta @ vs, axis=0)
    i = int(np.argmax(norms))
    out = oracle.fit_anchor(delta[None], 1)
    assert math.sqrt(out["eig"][0, 0]) == pytest.approx(norms[i], rel=1e-9)
    v = vs[:, i] * (1 if abs(vs[0, i]) >= abs(vs[1, i]) and vs[0, i] > 0 or
                    abs(vs[1, i]) > abs(vs[0, i]) and vs[1, i] > 0 else -1)
    np.testing.assert_allclose(out["W"][0, 0], v, atol=2e-5)
    # the smallest one minimises it
    assert math.sqrt(out["eig"][0, 1]) == pytest.approx(norms.min(), rel=1e-9)


def test_power_iteration_agrees_on_top_pair():
    rng = np.random.default_rng(6)
    delta = rng.standard_normal((30, 8)) @ np.diag([5, 2, 1, 1, 0.5, 0.5, 0.2, 0.1])
    v = np.ones(8)
    for _ in range(2000):
        # independent route: iterate with delta^T (delta v) without forming delta^T delta
        v = delta.T @ (delta @ v)
        v /= np.linalg.norm(v)
    lam = float(v @ (delta.T @ (delta @ v)))
    out = oracle.fit_anchor(delta[None], 1)
    assert out["eig"][0, 0] == pytest.approx(lam, rel=1e-12)
    v = v if v[np.argmax(np.abs(v))] > 0 else -v
    np.testing.assert_allclose(out["W"][0, 0], v, atol=1e-9)


@pytest.mark.parametrize("case", json.load(open(os.path.join(GOLDEN, "effective_rank.json")))["cases"])
def test_effective_rank_planted_closed_form(case):
    rho, r, energy, k = case["rho"], case["r"], case["energy"], case["k_eff"]
    lam = (3.0 * rho ** np.arange(r)) ** 2
    assert int(oracle.effective_rank(lam, energy)) == k
    # bracketing fractions of the geometric series
    frac = lambda kk: (1 - rho ** (2 * kk)) / (1 - rho ** (2 * r))  # noqa: E731
    assert frac(k - 1) == pytest.approx(case["frac_below"], abs=1e-4)
    assert frac(k) == pytest.approx(case["frac_at"], abs=1e-4)
    # padded with zero eigenvalues (d > r) the answer does not change
    assert int(oracle.effective_rank(np.concatenate([lam, np.zeros(96)]), energy)) == k
    # and it is the same through the fit of a planted delta with that spectrum
    rng = np.random.default_rng(r)
    _, _, delta = _planted(rng, 4 * r + 8, r + 4, 3.0 * rho ** np.arange(r))
    assert int(oracle.fit_anchor(delta[None], min(r, 4), energy)["k_eff"][0]) == k


def test_effective_rank_edges():
    assert int(oracle.effective_rank(np.zeros(5))) == 0
    assert int(oracle.effective_rank(np.array([9.0, 1.0]))) == 1  # exactly 90%: "at least"
    assert int(oracle.effective_rank(np.array([1.0, 9.0]))) == 1  # sorted first
    assert int(oracle.effective_rank(np.array([8.9, 1.1]))) == 2
    assert int(oracle.effective_rank(np.array([1.0, 1.0, 1.0, 1.0]), 1.0)) == 4
    assert int(oracle.effective_rank(np.array([5.0, -1e-9, 0.0]))) == 1  # negative round-off clamps
    np.testing.assert_array_equal(oracle.effective_rank(np.array([[9.0, 1.0], [1.0, 1.0]])), [1, 2])


def test_fit_rank_above_matrix_rank_and_wide_delta():
    rng = np.random.default_rng(3)
    delta = rng.standard_normal((3, 8))  # T < d: at most 3 nonzero eigenvalues
    out = oracle.fit_anchor(delta[None], 5)
    assert out["U"].shape == (1, 3, 5) and out["W"].shape == (1, 5, 8)
    np.testing.assert_allclose(out["eig"][0, 3:], 0.0)
    np.testing.assert_allclose(out["U"][0] @ out["W"][0], delta, atol=1e-13)
