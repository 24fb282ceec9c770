"""Pins of the oracle's online anchor pool (select_anchors, correct_pooled, pool_insert):
hand-worked selections, reduction to the plain correction when the pool holds exactly the
anchors, brute force, first-in first-out insertion and exact recovery after an insertion."""
import math

import numpy as np

import oracle
from test_oracle_correct import _brute_correct


def test_select_anchors_hand_cases():
    s = np.array([[0.1, 0.9, 0.5, 0.9, -0.3],   # tie 0.9: slot 1 before slot 3
                  [0.2, 0.7, 0.0, 0.0, 0.0],    # only 2 valid slots (A = 3)
                  [0.4, 0.4, 0.4, 0.4, 0.4],    # empty pool
                  [0.3, np.nan, 0.8, 0.1, 0.0]])  # NaN among the valid slots
    count = np.array([5, 2, 0, 4])
    slots, w, score = oracle.select_anchors(s, count, 3)
    np.testing.assert_array_equal(slots[0], [1, 3, 2])
    e = [math.exp(0.0), math.exp(0.0), math.exp(0.5 - 0.9)]
    np.testing.assert_allclose(w[0], np.array(e) / sum(e), rtol=1e-15)
    assert score[0] == 0.9
    np.testing.assert_array_equal(slots[1], [1, 0, 1])  # unused position repeats the best slot
    e = [1.0, math.exp(0.2 - 0.7)]
    np.testing.assert_allclose(w[1], [e[0] / sum(e), e[1] / sum(e), 0.0], rtol=1e-15)
    assert score[1] == 0.7  # slots past count are ignored, even with higher scores
    assert score[2] == -np.inf and np.all(w[2] == 0)  # empty: falls back at any tau
    np.testing.assert_array_equal(slots[3], [2, 0, 3])  # NaN ranks last ...
    assert np.isnan(score[3])  # ... but makes the score NaN (fallback)


def _pool(rng, L, H, Vc, T, d, r):
    return {"desc": rng.standard_normal((L, H, Vc, 2 * d)),
            "U": rng.standard_normal((2, L, H, Vc, T, r)) * 0.3,
            "W": rng.standard_normal((2, L, H, Vc, r, d)) * 0.3,
            "count": np.full((L, H), Vc), "head": np.zeros((L, H), dtype=np.int64)}


def test_full_pool_of_A_anchors_is_the_plain_correction():
    """With V = A and a full pool every slot is selected, in score order: the weighted sum
    does not depend on the order, so the result is ``correct`` on the same anchors."""
    rng = np.random.default_rng(21)
    L, H, T, d, A, r = 2, 2, 5, 4, 3, 2
    K = rng.standard_normal((L, H, T, d))
    V = rng.standard_normal((L, H, T, d))
    p = _pool(rng, L, H, A, T, d, r)
    a = oracle.correct_pooled(K, V, p, A, -0.05, "f32")
    b = oracle.correct(K, V, p["desc"], p["U"], p["W"], -0.05, "f32")
    np.testing.assert_array_equal(a["mask"], b["mask"])
    np.testing.assert_allclose(a["K_exact"], b["K_exact"], rtol=0, atol=1e-13)
    np.testing.assert_allclose(a["V_exact"], b["V_exact"], rtol=0, atol=1e-13)
    np.testing.assert_allclose(np.sort(a["w"], -1), np.sort(b["w"], -1), rtol=1e-14)


def test_pooled_correction_brute_force_on_the_selected_slots():
    rng = np.random.default_rng(22)
    L, H, T, d, Vc, A, r = 1, 3, 4, 3, 5, 2, 2
    K = rng.standard_normal((L, H, T, d))
    V = rng.standard_normal((L, H, T, d))
    p = _pool(rng, L, H, Vc, T, d, r)
    p["count"] = np.array([[5, 3, 1]])
    res = oracle.correct_pooled(K, V, p, A, -1.0, "f32")
    for h in range(H):
        sl = res["slots"][0, h]
        n = p["count"][0, h]
        # brute force: the plain correction over the selected slots, with their weights
        bk, bv, _ = _brute_correct(K[:, h:h + 1], V[:, h:h + 1],
                                   p["desc"][:, h:h + 1][:, :, sl[: min(A, n)]],
                                   p["U"][:, :, h:h + 1][:, :, :, sl[: min(A, n)]],
                                   p["W"][:, :, h:h + 1][:, :, :, sl[: min(A, n)]], -1.0)
        np.testing.assert_allclose(res["K_exact"][:, h:h + 1], bk, rtol=0, atol=1e-12)
        np.testing.assert_allclose(res["V_exact"][:, h:h + 1], bv, rtol=0, atol=1e-12)
        # the selected slots are the best valid ones
        sc = res["s"][0, h, :n]
        assert set(sl[: min(A, n)]) == set(np.argsort(-sc, kind="stable")[: min(A, n)])


def test_pool_insert_is_first_in_first_out():
    rng = np.random.default_rng(23)
    L, H, T, d, Vc, r = 1, 2, 3, 4, 3, 2
    st = {"desc": np.zeros((L, H, Vc, 2 * d)), "U": np.zeros((2, L, H, Vc, T, r)),
          "W": np.zeros((2, L, H, Vc, r, d)), "count": np.zeros((L, H), dtype=np.int64),
          "head": np.zeros((L, H), dtype=np.int64)}
    for i in range(5):
        U = np.full((2, L, H, T, r), float(i + 1))
        W = np.full((2, L, H, r, d), -float(i + 1))
        q = np.full((L, H, 2 * d), 10.0 * (i + 1))
        mask = np.array([[1, i % 2]], dtype=np.uint8)  # segment 1 inserts on odd requests
        new = oracle.pool_insert(st, mask, U, W, q, "bf16")
        assert np.all(st["count"] <= Vc)  # the input state is left as it was
        st = new
    # segment 0 took 5 insertions into 3 slots: anchors 4, 5, 3 (slot order), 3 the oldest
    np.testing.assert_array_equal(st["U"][0, 0, 0, :, 0, 0], [4.0, 5.0, 3.0])
    np.testing.assert_array_equal(st["W"][1, 0, 0, :, 0, 0], [-4.0, -5.0, -3.0])
    np.testing.assert_array_equal(st["desc"][0, 0, :, 0], [40.0, 50.0, 30.0])
    assert st["count"][0, 0] == 3 and st["head"][0, 0] == 2
    # segment 1 took the odd requests 2 and 4
    np.testing.assert_array_equal(st["U"][0, 0, 1, :, 0, 0], [2.0, 4.0, 0.0])
    assert st["count"][0, 1] == 2 and st["head"][0, 1] == 2


def test_pool_insert_rounds_factors_to_the_cache_dtype_once():
    L, H, T, d, Vc, r = 1, 1, 2, 2, 2, 1
    st = {"desc": np.zeros((L, H, Vc, 2 * d)), "U": np.zeros((2, L, H, Vc, T, r)),
          "W": np.zeros((2, L, H, Vc, r, d)), "count": np.zeros((L, H), dtype=np.int64),
          "head": np.zeros((L, H), dtype=np.int64)}
    x = 1.0 + 2.0 ** -8  # halfway between two bf16 values: ties to even gives 1.0
    y = 1.0 + 3 * 2.0 ** -8  # halfway: rounds up to 1 + 2^-6
    U = np.full((2, L, H, T, r), x)
    W = np.full((2, L, H, r, d), y)
    st = oracle.pool_insert(st, np.ones((1, 1)), U, W, np.full((1, 1, 4), 1.0 + 2.0 ** -30),
                            "bf16")
    assert st["U"][0, 0, 0, 0, 0, 0] == 1.0
    assert st["W"][0, 0, 0, 0, 0, 0] == 1.0 + 2.0 ** -6
    assert st["desc"][0, 0, 0, 0] == 1.0  # descriptors are float32


def test_insert_then_correct_recovers_the_observed_cache():
    """A fallback segment's fitted anchor, inserted with the reused cache's descriptor, makes
    the next request on the same reused cache match it with cosine 1 and recover the exact
    cache (planted rank-r deviation, fp64)."""
    rng = np.random.default_rng(24)
    L, H, T, d, Vc, A, r = 1, 2, 12, 6, 4, 2, 2
    K = rng.standard_normal((L, H, T, d))
    V = rng.standard_normal((L, H, T, d))
    DK = rng.standard_normal((L, H, T, r)) @ rng.standard_normal((L, H, r, d))
    DV = rng.standard_normal((L, H, T, r)) @ rng.standard_normal((L, H, r, d))
    st = {"desc": np.zeros((L, H, Vc, 2 * d)), "U": np.zeros((2, L, H, Vc, T, r)),
          "W": np.zeros((2, L, H, Vc, r, d)), "count": np.zeros((L, H), dtype=np.int64),
          "head": np.zeros((L, H), dtype=np.int64)}
    first = oracle.correct_pooled(K, V, st, A, 0.5, "f32")
    np.testing.assert_array_equal(first["mask"], 1)  # empty pools fall back
    delta = np.concatenate([DK, DV]).reshape(2 * L * H, T, d)
    fit = oracle.fit_anchor(delta, r)
    st = oracle.pool_insert(st, first["mask"], fit["U"].reshape(2, L, H, T, r),
                            fit["W"].reshape(2, L, H, r, d), first["q"], "f32")
    second = oracle.correct_pooled(K, V, st, A, 0.5, "f32")
    np.testing.assert_array_equal(second["mask"], 0)
    np.testing.assert_allclose(second["score"], 1.0, atol=1e-6)
    # the float32 storage of the factors bounds the recovery error
    assert oracle.rel_frobenius(second["K_exact"], K + DK) < 1e-6
    assert oracle.rel_frobenius(second["V_exact"], V + DV) < 1e-6
