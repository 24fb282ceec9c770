"""Pins of the oracle's non-chained correction (fanout) and of the error measures of the
listing's Fig. 3 (error normalised by the target, per layer and per agent) and Fig. 7(b)
(reconstruction error against the retained rank): brute force, closed forms, exact
recovery and Eckart-Young through an explicit reconstruction."""
import math

import numpy as np
import pytest

import oracle
from test_oracle_correct import _brute_correct


def _planted_factors(rng, L, H, T, d, r, scale):
    """U [L,H,T,r], W [L,H,r,d] with orthonormal W rows, and their product."""
    U = rng.standard_normal((L, H, T, r)) * scale
    W = np.empty((L, H, r, d))
    for l in range(L):
        for h in range(H):
            q, _ = np.linalg.qr(rng.standard_normal((d, r)))
            W[l, h] = q.T
    return U, W, U @ W


# ---------------------------------------------------------------------------- fanout


def _targets(rng, n, L, H, T, d, A, r):
    out = []
    for _ in range(n):
        out.append({
            "desc": rng.standard_normal((L, H, A, 2 * d)),
            "U": rng.standard_normal((2, L, H, A, T, r)) * 0.3,
            "W": rng.standard_normal((2, L, H, A, r, d)) * 0.3,
        })
    return out


def test_fanout_is_the_brute_force_correction_of_one_source_per_agent():
    rng = np.random.default_rng(11)
    L, H, T, d, A, r = 1, 2, 3, 4, 2, 2
    K = rng.standard_normal((L, H, T, d))
    V = rng.standard_normal((L, H, T, d))
    tg = _targets(rng, 3, L, H, T, d, A, r)
    # one target's first segment is forced below tau, with a fallback cache
    tg[1]["desc"][0, 0] = -np.concatenate([K[0, 0].mean(0), V[0, 0].mean(0)])[None].repeat(A, 0)
    tg[1]["K_fb"] = rng.standard_normal((L, H, T, d))
    tg[1]["V_fb"] = rng.standard_normal((L, H, T, d))
    K0, V0 = K.copy(), V.copy()
    res = oracle.fanout(K, V, tg, 0.1, "f32")
    assert len(res) == 3
    np.testing.assert_array_equal(K, K0)  # the reference is never modified
    np.testing.assert_array_equal(V, V0)
    for t, out in zip(tg, res):
        bk, bv, bm = _brute_correct(K, V, t["desc"], t["U"], t["W"], 0.1,
                                    t.get("K_fb"), t.get("V_fb"))
        np.testing.assert_array_equal(out["mask"], bm)
        np.testing.assert_allclose(out["K_exact"], bk, rtol=0, atol=1e-12)
        np.testing.assert_allclose(out["V_exact"], bv, rtol=0, atol=1e-12)
    assert res[1]["mask"][0, 0] == 1
    np.testing.assert_array_equal(res[1]["K_exact"][0, 0], tg[1]["K_fb"][0, 0])
    # every agent matched the same pooled descriptor of the reference
    for out in res:
        np.testing.assert_array_equal(out["q"], res[0]["q"])


def test_fanout_recovers_every_agent_exactly_with_its_planted_anchor():
    """Agent j's exact cache is C + U_j W_j; with that single anchor (A = 1, so w = 1) the
    non-chained correction of the context-free reference C gives agent j's cache."""
    rng = np.random.default_rng(12)
    L, H, T, d, r = 2, 2, 16, 8, 3
    CK = rng.standard_normal((L, H, T, d))
    CV = rng.standard_normal((L, H, T, d))
    tg, exact = [], []
    for _ in range(3):
        UK, WK, DK = _planted_factors(rng, L, H, T, d, r, 0.5)
        UV, WV, DV = _planted_factors(rng, L, H, T, d, r, 0.5)
        q = oracle.pool(CK, CV)
        tg.append({"desc": q[:, :, None, :], "U": np.stack([UK, UV])[:, :, :, None],
                   "W": np.stack([WK, WV])[:, :, :, None]})
        exact.append((CK + DK, CV + DV))
    res = oracle.fanout(CK, CV, tg, 0.5, "f32")
    for out, (EK, EV) in zip(res, exact):
        assert out["mask"].sum() == 0
        np.testing.assert_allclose(out["w"], 1.0)
        assert oracle.rel_frobenius(out["K_exact"], EK) < 1e-14
        assert oracle.rel_frobenius(out["V_exact"], EV) < 1e-14


def test_fanout_of_one_agent_is_the_first_chain_edge():
    rng = np.random.default_rng(13)
    L, H, T, d, A, r = 1, 3, 5, 4, 3, 2
    K = oracle.round_to_bf16(rng.standard_normal((L, H, T, d)))
    V = oracle.round_to_bf16(rng.standard_normal((L, H, T, d)))
    tg = _targets(rng, 1, L, H, T, d, A, r)
    a = oracle.fanout(K, V, tg, -0.2, "bf16")[0]
    b = oracle.chain(K, V, tg, -0.2, "bf16")[0]
    for key in ("K_out", "V_out", "mask", "w"):
        np.testing.assert_array_equal(a[key], b[key])


# ---------------------------------------------------------------------------- Fig. 3 error


def test_segment_error_brute_force():
    rng = np.random.default_rng(14)
    L, H, T, d = 2, 3, 4, 5
    X = rng.standard_normal((L, H, T, d))
    R = rng.standard_normal((L, H, T, d))
    e, r = oracle.segment_error(X, R)
    assert e.shape == (L, H) and r.shape == (L, H)
    for l in range(L):
        for h in range(H):
            se = sum((X[l, h, t, c] - R[l, h, t, c]) ** 2 for t in range(T) for c in range(d))
            sr = sum(R[l, h, t, c] ** 2 for t in range(T) for c in range(d))
            assert math.isclose(e[l, h], se, rel_tol=1e-13)
            assert math.isclose(r[l, h], sr, rel_tol=1e-13)


def test_segment_error_closed_forms():
    rng = np.random.default_rng(15)
    L, H, T, d = 2, 2, 7, 3
    R = rng.standard_normal((L, H, T, d))
    e, r = oracle.segment_error(R, R)
    np.testing.assert_array_equal(e, 0.0)
    e, r = oracle.segment_error(np.zeros_like(R), R)
    np.testing.assert_allclose(e, r, rtol=1e-15)  # error of the zero cache = ||ref||^2
    e, _ = oracle.segment_error(2.0 * R, R)
    np.testing.assert_allclose(e, r, rtol=1e-15)
    e, _ = oracle.segment_error(R + 0.25, R)  # a constant offset c gives c^2 T d
    np.testing.assert_allclose(e, 0.0625 * T * d, rtol=1e-12)


def test_layer_error_hand_values():
    err = np.array([[1.0, 3.0], [0.0, 0.0], [2.0, 0.0]])
    ref = np.array([[8.0, 8.0], [5.0, 0.0], [0.0, 0.0]])
    le = oracle.layer_error(err, ref)
    np.testing.assert_allclose(le[:2], [0.5, 0.0])
    assert le[2] == math.sqrt(2.0)  # no reference energy: the absolute error
    # summing the per-layer sums gives the whole-tensor relative error of rel_frobenius
    rng = np.random.default_rng(16)
    X = rng.standard_normal((3, 2, 6, 4))
    R = rng.standard_normal((3, 2, 6, 4))
    e, r = oracle.segment_error(X, R)
    assert math.isclose(math.sqrt(e.sum() / r.sum()), oracle.rel_frobenius(X, R), rel_tol=1e-13)


# ---------------------------------------------------------------------------- Fig. 7(b)


def test_rank_error_curve_geometric_spectrum_closed_form():
    """sigma_i = rho^i (i < n): the tail of a geometric series gives
    e(k)^2 = rho^(2k) (1 - rho^(2(n-k))) / (1 - rho^(2n))."""
    rho, n = 0.9, 32
    lam = rho ** (2.0 * np.arange(n))
    c = oracle.rank_error_curve(lam)
    assert c.shape == (n + 1,)
    for k in range(n + 1):
        want = math.sqrt(rho ** (2 * k) * (1 - rho ** (2 * (n - k))) / (1 - rho ** (2 * n)))
        assert math.isclose(c[k], want, rel_tol=1e-12, abs_tol=1e-15)


def test_rank_error_curve_is_the_error_of_the_fitted_anchor():
    """Eckart-Young through an explicit reconstruction: the oracle's rank-k anchor U W leaves
    exactly the relative error the curve gives at k."""
    rng = np.random.default_rng(17)
    D = rng.standard_normal((2, 30, 8)) * np.array([4.0, 3.0, 2.5, 2.0, 1.0, 0.5, 0.3, 0.1])
    full = oracle.fit_anchor(D, 8)
    curve = oracle.rank_error_curve(full["eig"])
    for k in (1, 2, 3, 5, 8):
        f = oracle.fit_anchor(D, k)
        for m in range(2):
            rec = f["U"][m] @ f["W"][m]
            err = np.linalg.norm(D[m] - rec) / np.linalg.norm(D[m])
            assert math.isclose(err, curve[m, k], rel_tol=1e-9, abs_tol=1e-12)


def test_rank_error_curve_edges_and_effective_rank():
    lam = np.array([[0.5, 4.0, 1.0, 0.0], [0.0, 0.0, 0.0, 0.0]])
    c = oracle.rank_error_curve(lam)  # unsorted input is sorted descending
    np.testing.assert_allclose(c[0], np.sqrt([5.5, 1.5, 0.5, 0.0, 0.0]) / math.sqrt(5.5))
    np.testing.assert_array_equal(c[1], 0.0)  # zero delta: no error at any rank
    # the effective rank is the first k whose error^2 is at most 1 - energy
    rng = np.random.default_rng(18)
    for _ in range(20):
        lam = np.sort(rng.exponential(size=16))[::-1] ** 3
        cur = oracle.rank_error_curve(lam)
        k = int(oracle.effective_rank(lam, 0.9))
        assert cur[k] ** 2 <= 0.1 + 1e-12 and cur[k - 1] ** 2 > 0.1 - 1e-12


@pytest.mark.parametrize("n", [1, 5])
def test_rank_error_curve_monotone(n):
    rng = np.random.default_rng(19 + n)
    c = oracle.rank_error_curve(rng.random((4, n)))
    assert np.all(np.diff(c, axis=-1) <= 1e-15)
    np.testing.assert_allclose(c[:, 0], 1.0)
    np.testing.assert_array_equal(c[:, -1], 0.0)
