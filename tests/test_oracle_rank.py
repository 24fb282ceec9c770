"""Pins of the oracle's matching on rank-r_C cache representations (rank_descriptor,
rank_scores, correct_rank): hand-worked factors, closed forms, invariances and brute force."""
import json
import math
import os

import numpy as np
import pytest

import oracle
from conftest import GOLDEN


def _ev(x: str) -> float:
    return float(eval(x, {"sqrt": math.sqrt, "exp": math.exp}))  # hand-written fixture values


@pytest.mark.parametrize("case", json.load(open(os.path.join(GOLDEN, "rank_matching_hand.json")))["cases"])
def test_rank_scores_hand_cases(case):
    Fq = np.array([case["Fq_K"], case["Fq_V"]], dtype=np.float64)[:, None, None]
    Fa = np.array([case["Fa_K"], case["Fa_V"]], dtype=np.float64)[:, None, None]
    s = oracle.rank_scores(Fq, Fa)[0, 0]
    np.testing.assert_allclose(s, [_ev(v) for v in case["s"]], rtol=1e-14, atol=1e-15)


def _rand_cache(rng, L, H, T, d, rank=None):
    X = rng.standard_normal((L, H, T, d))
    if rank is not None:
        X = rng.standard_normal((L, H, T, rank)) @ rng.standard_normal((L, H, rank, d))
    return X


def test_descriptor_gram_closed_forms():
    rng = np.random.default_rng(1)
    K = _rand_cache(rng, 2, 2, 40, 6)
    V = _rand_cache(rng, 2, 2, 40, 6) * 3.0
    # r_C = d: F^T F is the whole second-moment matrix X^T X
    out = oracle.rank_descriptor(K, V, 6)
    for x, X in enumerate((K, V)):
        for l in range(2):
            for h in range(2):
                F = out["F"][x, l, h]
                np.testing.assert_allclose(F.T @ F, X[l, h].T @ X[l, h], rtol=1e-11, atol=1e-10)
    # r_C < d: F^T F is the best rank-r_C approximation; its trace is the top-r_C energy
    out3 = oracle.rank_descriptor(K, V, 3)
    F = out3["F"][0, 1, 0]
    G = K[1, 0].T @ K[1, 0]
    lam = np.sort(np.linalg.eigvalsh(G))[::-1]
    np.testing.assert_allclose(np.trace(F.T @ F), lam[:3].sum(), rtol=1e-12)
    np.testing.assert_allclose(np.sort(np.linalg.eigvalsh(F.T @ F))[::-1][:3], lam[:3], rtol=1e-11)
    # rows are orthogonal with squared norms lambda_1 >= lambda_2 >= ...
    np.testing.assert_allclose(F @ F.T, np.diag(lam[:3]), rtol=1e-11, atol=1e-9)


def test_descriptor_invariant_to_token_order_and_planted_rank():
    rng = np.random.default_rng(2)
    K = _rand_cache(rng, 1, 2, 30, 5, rank=2)
    V = _rand_cache(rng, 1, 2, 30, 5)
    perm = rng.permutation(30)
    a = oracle.rank_descriptor(K, V, 4)
    b = oracle.rank_descriptor(K[:, :, perm], V[:, :, perm], 4)
    for x in range(2):
        for h in range(2):
            Fa, Fb = a["F"][x, 0, h], b["F"][x, 0, h]
            np.testing.assert_allclose(Fa.T @ Fa, Fb.T @ Fb, rtol=1e-10, atol=1e-10)
    # K has rank 2: rows 3 and 4 of its factor vanish and its effective rank is at most 2
    assert np.all(np.abs(a["F"][0, 0, :, 2:]) < 1e-10)
    assert np.all(a["k_eff"][0] <= 2)


def test_constant_rows_give_the_squared_pooled_cosine():
    """Rank-1 degenerate case: constant-row caches X = 1 k^T.  Their representation is
    sqrt(T)|k| k^, so the similarity of two such caches (V zero) is cos^2 of the rows, the
    square of the mean-pool cosine of the plain descriptor."""
    rng = np.random.default_rng(3)
    for _ in range(5):
        k1, k2 = rng.standard_normal(7), rng.standard_normal(7)
        T1, T2 = 11, 25
        K1 = np.tile(k1, (1, 1, T1, 1))
        K2 = np.tile(k2, (1, 1, T2, 1))
        Z1, Z2 = np.zeros_like(K1), np.zeros_like(K2)
        F1 = oracle.rank_descriptor(K1, Z1, 2)["F"]
        F2 = oracle.rank_descriptor(K2, Z2, 2)["F"]
        np.testing.assert_allclose(np.linalg.norm(F1[0, 0, 0, 0]), math.sqrt(T1) * np.linalg.norm(k1), rtol=1e-12)
        s = oracle.rank_scores(F1, F2[:, :, :, None])[0, 0, 0]
        q1, q2 = oracle.pool(K1, Z1)[0, 0], oracle.pool(K2, Z2)[0, 0]
        c = oracle.cosine_scores(q1[None], q2[None, None])[0, 0]
        np.testing.assert_allclose(s, c * c, rtol=1e-11)


def test_rank_scores_invariances():
    rng = np.random.default_rng(4)
    Fq = rng.standard_normal((2, 2, 3, 4, 9))
    Fa = rng.standard_normal((2, 2, 3, 5, 4, 9))
    s = oracle.rank_scores(Fq, Fa)
    assert np.all(s > 0) and np.all(s <= 1 + 1e-12)  # PSD matrices: cosine in [0, 1]
    # a rotation (or sign flip) of the factor rows, a scale of a factor: unchanged
    Q, _ = np.linalg.qr(rng.standard_normal((4, 4)))
    np.testing.assert_allclose(oracle.rank_scores(np.einsum("ij,xlhjd->xlhid", Q, Fq), Fa), s,
                               rtol=1e-11)
    np.testing.assert_allclose(oracle.rank_scores(Fq, -2.5 * Fa), s, rtol=1e-12)
    # the representation against itself scores 1; a permutation of anchors permutes s
    np.testing.assert_allclose(oracle.rank_scores(Fq, Fq[:, :, :, None]), 1.0, rtol=1e-12)
    perm = [3, 0, 4, 1, 2]
    np.testing.assert_allclose(oracle.rank_scores(Fq, Fa[:, :, :, perm]), s[..., perm], rtol=1e-13)


def test_rank_scores_brute_force_on_full_matrices():
    rng = np.random.default_rng(5)
    Fq = rng.standard_normal((2, 1, 2, 3, 6))
    Fa = rng.standard_normal((2, 1, 2, 4, 3, 6))
    s = oracle.rank_scores(Fq, Fa)
    for h in range(2):
        gq = np.concatenate([(Fq[x, 0, h].T @ Fq[x, 0, h]).ravel() for x in range(2)])
        for a in range(4):
            ga = np.concatenate([(Fa[x, 0, h, a].T @ Fa[x, 0, h, a]).ravel() for x in range(2)])
            want = float(gq @ ga) / (np.linalg.norm(gq) * np.linalg.norm(ga))
            assert s[0, h, a] == pytest.approx(want, rel=1e-12)


def test_correct_rank_is_correct_with_those_scores():
    rng = np.random.default_rng(6)
    L, H, T, d, A, r = 2, 2, 9, 4, 3, 2
    K, V = rng.standard_normal((L, H, T, d)), rng.standard_normal((L, H, T, d))
    U, W = rng.standard_normal((2, L, H, A, T, r)), rng.standard_normal((2, L, H, A, r, d))
    Fq = oracle.rank_descriptor(K, V, 2)["F"]
    Fa = np.stack([Fq + 0.3 * a * rng.standard_normal(Fq.shape) for a in range(A)], axis=3)
    out = oracle.correct_rank(K, V, Fq, Fa, U, W, 0.8, "f32")
    s = oracle.rank_scores(Fq, Fa)
    np.testing.assert_allclose(out["s"], s)
    # anchor 0 is the query itself: score 1, so nothing falls back at tau = 0.8
    np.testing.assert_allclose(out["score"], 1.0, rtol=1e-12)
    assert not out["mask"].any()
    # brute force of one segment
    w = np.exp(s[1, 0] - s[1, 0].max())
    w /= w.sum()
    want = K[1, 0] + sum(w[a] * U[0, 1, 0, a] @ W[0, 1, 0, a] for a in range(A))
    np.testing.assert_allclose(out["K_exact"][1, 0], want, rtol=1e-13)
    # tau above 1: everything falls back to the source
    fb = oracle.correct_rank(K, V, Fq, Fa, U, W, 1.5, "f32")
    assert fb["mask"].all()
    np.testing.assert_array_equal(fb["K_exact"], K)
